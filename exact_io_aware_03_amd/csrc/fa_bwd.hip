// Exact attention backward for gfx950, recomputing P from the saved logsumexp.
//
// Method (Lecture 21 notes, CMU 11-868, §2.6 and exercises 4-6): the forward keeps only O and
// L = m + log l per row. The backward rebuilds each tile's P = exp(scale*S - L), forms
// dV += P^T dO, dP = dO V^T, dS = P * (dP - D) with D = rowsum(dO * O) computed by a small
// pre-kernel (sum_k P_ik dP_ik = dO_i . O_i), dK += scale dS^T Q and dQ += scale dS K. The outer
// loop runs over K/V blocks so dK and dV stay on chip and only dQ is accumulated across
// workgroups with atomic adds (half the atomics of a query-outer order).
//
// gfx950 mapping: a workgroup owns 128 keys (32 per wave, one wave per SIMD) of one
// (batch, kv head) and walks the 64-row query blocks that can see them (causal: only blocks at
// or below the diagonal, longest task first), for every query head of the GQA group, as one
// flat sequence of steps. Per step:
//  * Q, dO (row-major) and L, D of the next step stream into the other half of a double
//    buffer with direct-to-LDS loads while this step computes;
//  * S = Q K^T and dP = dO V^T come out of the MFMA with one key per lane (K and V rows sit in
//    registers for the whole task), so P^T and dS^T feed the dV and dK products straight from
//    the accumulators (query rows relabelled as in the forward); the B operands of those
//    products (dO and Q with 8 consecutive rows per lane) are read transposed from the same
//    row-major tiles with ds_read_b64_tr_b16, one XOR swizzle serving both access patterns;
//  * dS^T goes to LDS with 16-byte stores and comes back transposed as the A operand of
//    dQ = dS K (K row-major in LDS for the whole task); each wave owns two 32x32 dQ tiles whose
//    rows map to coalesced fp32 global atomics.
// Two barriers per step: one after this step's tiles have landed, one after dS^T is complete.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;             // pre / post kernels
constexpr int kMainThreads = 512;         // main kernel: 8 waves, two per SIMD
constexpr int kWaves = kMainThreads / 64;
constexpr int BK = kBwdKeys;  // 128 keys per workgroup
constexpr int BQ = kBwdRows;  // 64 query rows per step

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Chunk swizzle of the row-major Q, dO and K tiles (16-byte chunks XOR-ed with a function of
// the row). Row reads (16 lanes, 16 rows, one logical chunk) need a bijection of the row's low
// 4 bits (d=128: 16 chunks per 256-byte row) or of bits 1-3 (d=64: two 128-byte rows per bank
// line); transposed reads (16 lanes, 4 consecutive rows x 32 bytes) need the 4 rows to differ in
// chunk bits 2-3. Swapping the two 2-bit halves of the row's low nibble does both at d=128.
template <int D>
__device__ __forceinline__ int t_swz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((row >> 1) & 7);
}
// dS^T tile [key][query], 128-byte rows.
__device__ __forceinline__ int ds_swz(int row) { return (row >> 1) & 7; }

template <int D>
struct BwdLds {
  static constexpr int ROW = D * 2;
  static constexpr int KT = BK * ROW;      // K or V, row-major [key][d]
  static constexpr int QT = BQ * ROW;      // one Q or dO tile, row-major [q][d]
  static constexpr int DST = BK * BQ * 2;  // dS^T, [key][q]
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = OFF_K + KT;
  static constexpr int OFF_Q = OFF_V + KT;          // Q[2]
  static constexpr int OFF_DO = OFF_Q + 2 * QT;     // dO[2]
  static constexpr int OFF_DS = OFF_DO + 2 * QT;
  static constexpr int OFF_L = OFF_DS + DST;        // L[2][BQ] fp32 (natural log)
  static constexpr int OFF_D = OFF_L + 2 * BQ * 4;  // D[2][BQ] fp32
  static constexpr int BYTES = OFF_D + 2 * BQ * 4;
  static constexpr int RR = 1024 / ROW;             // rows per 1 KiB direct-to-LDS load
  static constexpr int QDMA = QT / 1024 / kWaves;   // loads per wave per Q or dO tile
  static constexpr int KDMA = KT / 1024 / kWaves;   // loads per wave per K or V tile
  static constexpr int STEP_DMA = 2 * QDMA + 1;     // Q, dO and one of L (waves 0-3) or D (4-7)
  // fp32 dK/dV partials of the query-half-1 waves, reduced at the end through LDS
  static constexpr int RED = (kWaves / 2) * 2 * (D / 32) * 16 * 64 * 4;
  static_assert(RED <= BYTES, "reduction buffer");
};

// Raw buffer resource as four scalar words (base, stride 0, size, 32-bit untyped format).
__device__ __forceinline__ u32x4 dma_rsrc(const void* base, long bytes) {
  const unsigned long long p = (unsigned long long)base;
  u32x4 r;
  r[0] = (uint32_t)p;
  r[1] = (uint32_t)(p >> 32) & 0xffffu;
  r[2] = bytes <= 0 ? 0u : (bytes >= 0x7fffffffL ? 0x7fffffffu : (uint32_t)bytes);
  r[3] = 0x00020000u;
  return r;
}

// Wave-wide direct-to-LDS loads: lane i's 16 (or 4) bytes land at dst + 16 i (4 i). Inline asm
// so that the compiler does not wait for these loads before unrelated LDS reads; completion is
// ordered explicitly with s_waitcnt vmcnt before the barrier that publishes a tile.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is written by the asm itself
__device__ __forceinline__ void lds_dma16(const u32x4& r, char* dst, int voff) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(size_t)((__attribute__((address_space(3))) char*)dst));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const u32x4& r, char* dst, int voff) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(size_t)((__attribute__((address_space(3))) char*)dst));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Scheduling fence: no instruction moves across it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Wait until at most N vector-memory operations of this wave are pending and its LDS accesses
// are done, then the workgroup barrier. The empty asm statements keep the compiler from moving
// memory accesses across.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// The same for LDS only: vector-memory operations (prefetches, atomics) stay in flight.
__device__ __forceinline__ void lds_barrier() { wait_vm_barrier<63>(); }

// This wave's share of the direct-to-LDS loads of `rows` rows of a row-major [*, D] bf16 tensor
// into a swizzled LDS tile: load p of wave w fills 1 KiB (region kWaves*p + w), lane i landing
// on row RR*region + i/KCH, physical chunk i%KCH, and fetching the logical chunk the swizzle
// puts there. Rows at or past `valid_rows` read as zero.
template <int D, int NLOAD>
__device__ __forceinline__ void dma_rows(char* dst, const uint16_t* src, long row_stride, int valid_rows) {
  using L = BwdLds<D>;
  constexpr int KCH = D / 8;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const u32x4 r = dma_rsrc(src, ((long)(valid_rows - 1) * row_stride + D) * 2);
#pragma unroll
  for (int p = 0; p < NLOAD; ++p) {
    const int region = kWaves * p + w;
    const int row = L::RR * region + lane / KCH, pc = lane % KCH;
    const int voff = (int)((row * row_stride + ((pc ^ t_swz<D>(row)) * 8)) * 2);
    lds_dma16(r, dst + region * 1024, voff);
  }
}

// A operand of a transposed product read from a row-major LDS tile with two
// ds_read_b64_tr_b16: lane l receives column c0 + l%32 (c0 = 32*cb) and the 8 consecutive rows
// 16ks + 8(l/32) .. +7. In each 16-lane group, source lane s points at row r0 + s/4,
// columns 16((l/16)%2) + 4(s%4) .. +3 of the block.
template <int ROWB, typename Swz>
__device__ __forceinline__ bf16x8 tr_frag(const char* base, int ks, int cb, int lane, Swz swz) {
  const int s = lane & 15, g = lane >> 4;
  i16x4 r[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int row = 16 * ks + 8 * (g >> 1) + 4 * rd + (s >> 2);
    const int col_b = (32 * cb + 16 * (g & 1) + 4 * (s & 3)) * 2;  // byte column
    const int off = row * ROWB + (((col_b >> 4) ^ swz(row)) << 4) + (col_b & 15);
    r[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
  }
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 c = __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// D = rowsum(dO * O) per (batch, head, row) and a zeroed fp32 dQ accumulator. One wave per row.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*Nq + i)*Hq + h
  const int lane = threadIdx.x & 63;
  if (row >= a.B * a.Nq * a.Hq) return;
  const int h = row % a.Hq, i = (row / a.Hq) % a.Nq, b = row / (a.Hq * a.Nq);
  const uint16_t* op = (const uint16_t*)a.o + (long)row * D;
  const uint16_t* gp = (const uint16_t*)a.dout + (long)row * D;
  float s = 0.f;
  for (int e = lane; e < D / 2; e += 64) {
    const uint32_t ow = ((const uint32_t*)op)[e], gw = ((const uint32_t*)gp)[e];
    s = fmaf(bf16_lo(ow), bf16_lo(gw), s);
    s = fmaf(bf16_hi(ow), bf16_hi(gw), s);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) a.dvec[((long)b * a.Hq + h) * a.Nq + i] = s;
  float* acc = a.dq_acc + (long)row * D;
  for (int e = lane; e < D; e += 64) acc[e] = 0.f;
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_post_kernel(BwdArgs a, long n) {
  for (long e = (long)blockIdx.x * kThreads + threadIdx.x; e < n; e += (long)gridDim.x * kThreads)
    ((__bf16*)a.dq)[e] = (__bf16)(a.dq_acc[e] * a.scale);
}

template <int D>
__global__ __launch_bounds__(kMainThreads, 1) void bwd_main_kernel(BwdArgs a) {
  using L = BwdLds<D>;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int NT = 2 * DB;        // 32x32 dQ tiles per step (one per wave while they last)
  constexpr int NA = 16;            // dQ atomic instructions per tile
  static_assert(NA + L::STEP_DMA < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  char* kl = smem + L::OFF_K;
  char* vl = smem + L::OFF_V;
  char* dsl = smem + L::OFF_DS;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int slice = wave & 3;   // 32-key slice of the block
  const int qhalf = wave >> 2;  // 32-row half of each 64-row query block
  const bool dq_tile = wave < NT;
  // causal: kv block 0 sees every query block; dispatch order is longest first over all
  // (batch, kv head) pairs. Non-causal: XCD-contiguous ranges of one (batch, kv head).
  int bhk, j;
  if (a.causal) {
    const int n_bhk = a.n_tasks / a.n_kvblk;
    j = (int)blockIdx.x / n_bhk;
    bhk = (int)blockIdx.x % n_bhk;
  } else {
    const int task = xcd_contiguous_task(blockIdx.x, a.n_tasks);
    bhk = task / a.n_kvblk;
    j = task % a.n_kvblk;
  }
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int kv0 = j * BK;
  const int kw0 = kv0 + slice * 32;  // this wave's keys
  const int key = kw0 + l32;         // this lane's key
  const uint16_t* kp = (const uint16_t*)a.k + (long)b * a.Nk * a.k_row + hk * D;
  const uint16_t* vp = (const uint16_t*)a.v + (long)b * a.Nk * a.k_row + hk * D;

  // K and V rows of the block, row-major in LDS: B operands of S = Q K^T and dP = dO V^T
  // (row reads) and of dQ = dS K (transposed reads)
  dma_rows<D, L::KDMA>(kl, kp + (long)kv0 * a.k_row, a.k_row, a.Nk - kv0);
  dma_rows<D, L::KDMA>(vl, vp + (long)kv0 * a.k_row, a.k_row, a.Nk - kv0);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  const int n_qblk = (a.Nq + BQ - 1) / BQ;
  const int qb_first = a.causal ? kv0 / BQ : 0;
  const int per_head = n_qblk - qb_first;
  const int n_steps = a.G * per_head;

  // Issue the loads of step st (query head hk*G + st/per_head, block qb_first + st%per_head)
  // into buffer st&1: Q and dO tiles, and L (waves 0-3) or D (waves 4-7).
  auto issue_step = [&](int st) {
    const int hq = hk * a.G + st / per_head, q0 = (qb_first + st % per_head) * BQ;
    const int buf = st & 1;
    const long qoff = ((long)b * a.Nq + q0) * a.q_row + hq * D;
    dma_rows<D, L::QDMA>(smem + L::OFF_Q + buf * L::QT, (const uint16_t*)a.q + qoff, a.q_row, a.Nq - q0);
    dma_rows<D, L::QDMA>(smem + L::OFF_DO + buf * L::QT, (const uint16_t*)a.dout + qoff, a.q_row, a.Nq - q0);
    const long loff = ((long)b * a.Hq + hq) * a.Nq + q0;
    const long lbytes = (long)min(BQ, a.Nq - q0) * 4;
    if (qhalf == 0) lds_dma4(dma_rsrc(a.lse + loff, lbytes), smem + L::OFF_L + buf * BQ * 4, lane * 4);
    else lds_dma4(dma_rsrc(a.dvec + loff, lbytes), smem + L::OFF_D + buf * BQ * 4, lane * 4);
  };

  issue_step(0);
  bool prev_full = true;  // the previous step issued all of this wave's dQ atomics
  for (int st = 0; st < n_steps; ++st) {
    const int hq = hk * a.G + st / per_head, q0 = (qb_first + st % per_head) * BQ;
    const bool has_next = st + 1 < n_steps;
    if (has_next) issue_step(st + 1);
    // This step's loads (and, at st = 0, the K/V tiles) are complete once at most the loads
    // issued after them are pending: the previous step's dQ atomics (when this wave issued
    // all of them) and the next step's tiles.
    const bool after_atomics = st > 0 && prev_full && dq_tile;
    if (has_next) {
      if (after_atomics) wait_vm_barrier<NA + L::STEP_DMA>();
      else wait_vm_barrier<L::STEP_DMA>();
    } else {
      if (after_atomics) wait_vm_barrier<NA>();
      else wait_vm_barrier<0>();
    }
    // LDS addresses are recomputed each step from a pinned copy of the lane index instead of
    // being hoisted out of the loop: VALU time is cheap here, registers are not.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lh = ln >> 5, ll = ln & 31;
    const int buf = st & 1;
    const char* ql = smem + L::OFF_Q + buf * L::QT;
    const char* dol = smem + L::OFF_DO + buf * L::QT;
    const float* lls = (const float*)(smem + L::OFF_L + buf * BQ * 4);
    const float* dls = (const float*)(smem + L::OFF_D + buf * BQ * 4);

    // ---- S = Q K^T and dP = dO V^T for this wave's 32 rows x 32 keys ----
    // (causal blocks entirely above this wave's keys run too: their P is masked to zero)
    f32x16 s, g;
    zero16(s);
    zero16(g);
    {
      const int row = 32 * qhalf + swap_bits23(ll);  // A operand rows (relabelled)
      const int sw = t_swz<D>(row);
      const int kr = 32 * slice + ll;                // B operand: this lane's key row
      const int ksw = t_swz<D>(kr);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = row * L::ROW + (((2 * ks + lh) ^ sw) << 4);
        const int koff = kr * L::ROW + (((2 * ks + lh) ^ ksw) << 4);
        s = mfma_32x32x16(*(const bf16x8*)(ql + off), *(const bf16x8*)(kl + koff), s);
        g = mfma_32x32x16(*(const bf16x8*)(dol + off), *(const bf16x8*)(vl + koff), g);
      }
    }
    // register i holds query row 32qhalf + (i&7) + 8h + 16(i>>3) and key `key`: the 8 rows
    // (i&7) are consecutive, so L and D come in as 16-byte LDS reads.
    const int qw0 = q0 + 32 * qhalf;  // first row of this wave's half
    const bool need_mask = kw0 + 31 >= a.Nk || (a.causal && kw0 + 31 > qw0);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r0 = 32 * qhalf + 16 * hi + 8 * lh;
      const f32x4 la = *(const f32x4*)(lls + r0), lb = *(const f32x4*)(lls + r0 + 4);
      const f32x4 da = *(const f32x4*)(dls + r0), dbv = *(const f32x4*)(dls + r0 + 4);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int i = 8 * hi + x;
        const float lv = x < 4 ? la[x] : lb[x - 4], dvv = x < 4 ? da[x] : dbv[x - 4];
        float p = fast_exp2(fmaf(s[i], a.c, -lv * kLog2e));
        if (need_mask && (key >= a.Nk || (a.causal && key > q0 + r0 + x))) p = 0.f;
        s[i] = p;                   // P
        g[i] = p * (g[i] - dvv);  // dS
      }
    }
    // ---- dV += P^T dO, dK += dS^T Q over this wave's 32 rows (16 per step); dS^T to LDS ----
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kq = 2 * qhalf + kk;  // 16-row step within the 64-row block
      const int e = kk * 8;
      u32x4 pw, gw;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        pw[x] = pack_bf16x2(s[e + 2 * x], s[e + 2 * x + 1]);
        gw[x] = pack_bf16x2(g[e + 2 * x], g[e + 2 * x + 1]);
      }
      const int kc = 32 * slice + ll;
      *(u32x4*)(dsl + kc * (BQ * 2) + (((2 * kq + lh) ^ ds_swz(kc)) << 4)) = gw;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dv[db] = mfma_32x32x16(as_bf16x8(pw), tr_frag<L::ROW>(dol, kq, db, ln, t_swz<D>), dv[db]);
        dk[db] = mfma_32x32x16(as_bf16x8(gw), tr_frag<L::ROW>(ql, kq, db, ln, t_swz<D>), dk[db]);
      }
    }
    lds_barrier();  // dS^T complete

    // ---- dQ[64 x D] += dS[64 x 128] K[128 x D]; wave w owns tile (query half w%2, dims w/2) ----
    const bool full = q0 + BQ <= a.Nq;
    if (dq_tile) {
      const int qh = wave & 1, db = wave >> 1;
      f32x16 acc;
      zero16(acc);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks)
        acc = mfma_32x32x16(tr_frag<BQ * 2>(dsl, ks, qh, ln, ds_swz), tr_frag<L::ROW>(kl, ks, db, ln, t_swz<D>),
                            acc);
      // register i holds query row 32qh + 8(i/4) + 4h + i%4, dim 32db + l32
      float* dst = a.dq_acc + (((long)b * a.Nq + q0 + 32 * qh + 4 * h) * a.Hq + hq) * D + 32 * db + l32;
      const long rs = (long)a.Hq * D;
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) unsafeAtomicAdd(dst + (8 * (i >> 2) + (i & 3)) * rs, acc[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (q0 + 32 * qh + 8 * (i >> 2) + 4 * h + (i & 3) < a.Nq)
            unsafeAtomicAdd(dst + (8 * (i >> 2) + (i & 3)) * rs, acc[i]);
      }
    }
    prev_full = full;
  }
  __builtin_amdgcn_s_waitcnt(0);

  // ---- reduce the two query halves' partials; dK = scale * acc, dV = acc (bf16) ----
  // register i holds key kw0 + 8(i/4) + 4h + i%4, dim 32db + l32
  wait_vm_barrier<0>();  // every wave is done with the tiles: the LDS is free
  float* red = (float*)smem + (size_t)slice * (2 * DB * 16 * 64) + lane;
  if (qhalf == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        red[((2 * db) * 16 + i) * 64] = dk[db][i];
        red[((2 * db + 1) * 16 + i) * 64] = dv[db][i];
      }
  }
  wait_vm_barrier<0>();
  if (qhalf == 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = kw0 + 8 * (i >> 2) + 4 * h + (i & 3);
        const float dkv = dk[db][i] + red[((2 * db) * 16 + i) * 64];
        const float dvv = dv[db][i] + red[((2 * db + 1) * 16 + i) * 64];
        if (kk < a.Nk) {
          const long off = ((long)b * a.Nk + kk) * a.k_row + hk * D + 32 * db + l32;
          ((__bf16*)a.dk)[off] = (__bf16)(dkv * a.scale);
          ((__bf16*)a.dv)[off] = (__bf16)dvv;
        }
      }
  }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.Nq * a.Hq;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((rows + 3) / 4), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_main_kernel<D>), dim3(a.n_tasks), dim3(kMainThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long n = rows * D;
  const long blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((bwd_post_kernel<D>), dim3(blocks < 65536 ? blocks : 65536), dim3(kThreads), 0, s, a, n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, hipStream_t s) {
  return d == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace fa
