// Exact attention backward for gfx950, recomputing P from the saved logsumexp.
//
// Method (Lecture 21 notes, CMU 11-868, §2.6 and exercises 4-6): the forward keeps only O and
// L = m + log l per row. The backward rebuilds each tile's P = exp(scale*S - L), forms
// dV += P^T dO, dP = dO V^T, dS = P * (dP - D) with D = rowsum(dO * O) (sum_k P_ik dP_ik =
// dO_i . O_i), dK += scale dS^T Q and dQ += scale dS K.
//
// gfx950 mapping: two kernels, neither with atomics. The dQ kernel runs first and also writes
// D for its rows (it loads O and dO for them anyway); the dK/dV kernel reads D afterwards.
//  * dK/dV, key-block outer: a workgroup owns 128 keys of one (batch, kv head); its eight
//    waves (two per SIMD) are four 32-key slices x two 32-row halves of every 64-row query
//    block it walks (causal: only blocks at or below the diagonal, longest task first), for
//    every query head of the GQA group, as one flat sequence of steps. K and V sit in LDS for
//    the whole task; each step's Q, dO, L and D stream into the other half of a double buffer
//    with direct-to-LDS loads while the current step computes. S = Q K^T and dP = dO V^T come
//    out of the MFMA with one key per lane, so P^T and dS^T feed the dV and dK products
//    straight from the accumulators (query rows relabelled as in the forward); the B operands
//    (dO and Q, 8 consecutive rows per lane) are read transposed from the same row-major tiles
//    with ds_read_b64_tr_b16, one XOR swizzle serving both access patterns. The two row
//    halves' partial dK/dV are summed through LDS at the end.
//  * dQ, query-block outer (below): like the forward, with dQ in registers.
// Recomputing S and dP in the dQ kernel costs two extra products per tile; in exchange dQ is
// never read back and rewritten through fp32 atomics (one pass over an fp32 copy of dQ per key
// block), and the result is reproducible.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

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

template <int D>
struct BwdLds {
  static constexpr int ROW = D * 2;
  static constexpr int KT = BK * ROW;      // K or V block in MFMA fragment order
  static constexpr int QT = BQ * ROW;      // one Q or dO tile, row-major [q][d], swizzled
  // Q and dO first: their reads take the buffer offset as an instruction immediate (< 64 KiB)
  static constexpr int OFF_Q = 0;                   // Q[2]
  static constexpr int OFF_DO = OFF_Q + 2 * QT;     // dO[2]
  static constexpr int OFF_K = OFF_DO + 2 * QT;
  static constexpr int OFF_V = OFF_K + KT;
  static constexpr int OFF_L = OFF_V + KT;          // L[2][BQ] fp32 (natural log)
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

// Direct-to-LDS loads of a K or V block in MFMA fragment order: the 1 KiB region
// R = (D/16)*slice + ks holds at byte 16 l the 8 values that lane l feeds to the score product
// of 32-key slice `slice` and 16-dim step ks -- key 32 slice + l%32, dims 16 ks + 8(l/32) .. +7
// -- so those reads are lane-contiguous (no bank conflicts) at constant offsets from one
// per-lane base. Keys at or past `valid_rows` read as zero.
template <int D, int NLOAD>
__device__ __forceinline__ void dma_frag(char* dst, const uint16_t* src, long row_stride, int valid_rows) {
  constexpr int KS = D / 16;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const u32x4 r = dma_rsrc(src, ((long)(valid_rows - 1) * row_stride + D) * 2);
#pragma unroll
  for (int p = 0; p < NLOAD; ++p) {
    const int region = kWaves * p + w;
    const int row = 32 * (region / KS) + (lane & 31);
    const int voff = (int)((row * row_stride + 16 * (region % KS) + 8 * (lane >> 5)) * 2);
    lds_dma16(r, dst + region * 1024, voff);
  }
}

template <int N>
struct Const {
  static constexpr int value = N;
};

// DROP: the forward's dropout on P (Lecture 21 notes §2.8, exercise 4), its mask regenerated:
// dV takes P * Z / (1 - p), dP = (dO V^T) * Z / (1 - p), and D = rowsum(dO * O) still holds.
template <int D, bool DROP>
__global__ __launch_bounds__(kMainThreads, 1) void bwd_main_kernel(BwdArgs a) {
  using L = BwdLds<D>;
  constexpr int KS = D / 16, DB = D / 32;
  static_assert(L::STEP_DMA < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  char* kl = smem + L::OFF_K;
  char* vl = smem + L::OFF_V;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int slice = wave & 3;   // 32-key slice of the block
  const int qhalf = wave >> 2;  // 32-row half of each 64-row query block
  // causal: kv block 0 sees every query block; dispatch order is longest first, each XCD
  // keeping its own (batch, kv head) pairs. Non-causal: XCD-contiguous task ranges.
  int bhk, j;
  if (a.causal) {
    xcd_longest_first((int)blockIdx.x, a.n_tasks / a.n_kvblk, a.n_kvblk, bhk, j);
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

  // K and V of the block in LDS, in MFMA fragment order: B operands of S = Q K^T and dP = dO V^T
  dma_frag<D, L::KDMA>(kl, kp + (long)kv0 * a.k_row, a.k_row, a.Nk - kv0);
  dma_frag<D, L::KDMA>(vl, vp + (long)kv0 * a.k_row, a.k_row, a.Nk - kv0);

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

  // Per-lane LDS byte offsets, fixed for the whole task; the buffer, tensor and step parts of
  // every address are compile-time constants that go into the instructions' offset field.
  // Q / dO as A operands of S and dP: row 32 qhalf + relabelled l32, logical chunk 2 ks + h.
  int qoff[KS];
  {
    const int row = 32 * qhalf + swap_bits23(l32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qoff[ks] = row * L::ROW + (((2 * ks + h) ^ t_swz<D>(row)) << 4);
  }
  // dO / Q as transposed B operands of dV and dK (two ds_read_b64_tr_b16 per fragment): in each
  // 16-lane group, source lane s points at row r0 + s/4 of the 16-row step, columns
  // 32 db + 16((l/16)%2) + 4(s%4) .. +3; lane l receives column 32 db + l%32 and 8 consecutive
  // rows. The swizzle depends on the row's position within the 16-row step only.
  int troff[DB][2];
  {
    const int sl = lane & 15, g = lane >> 4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int rr = 8 * (g >> 1) + 4 * rd + (sl >> 2);
        const int col_b = (32 * db + 16 * (g & 1) + 4 * (sl & 3)) * 2;
        troff[db][rd] = (32 * qhalf + rr) * L::ROW + (((col_b >> 4) ^ t_swz<D>(rr)) << 4) + (col_b & 15);
      }
  }
  const int kvb = L::OFF_K + slice * KS * 1024 + lane * 16;  // K fragments; V at +KT
  const int lb = L::OFF_L + (32 * qhalf + 8 * h) * 4;        // L rows of this lane; D at +2BQ*4
  auto ld16 = [&](int off) { return *(const bf16x8*)(smem + off); };
  auto ld4f = [&](int off) { return *(const f32x4*)(smem + off); };
  auto tr8 = [&](int off0, int off1) {
    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + off0));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + off1));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // One step; the loop below is unrolled by two so the double-buffer index is a constant.
  auto step = [&](const int st, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int QB = L::OFF_Q + BUF * L::QT, GB = L::OFF_DO + BUF * L::QT;
    const int q0 = (qb_first + st % per_head) * BQ;
    // This step's loads (and, at st = 0, the K/V tiles) have landed, and every wave is done
    // with the previous step, whose buffer the next step's loads refill: issue them only now.
    wait_vm_barrier<0>();
    if (st + 1 < n_steps) issue_step(st + 1);

    // ---- S = Q K^T and dP = dO V^T for this wave's 32 rows x 32 keys ----
    // (causal blocks entirely above this wave's keys run too: their P is masked to zero)
    f32x16 s, g;
    zero16(s);
    zero16(g);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma_32x32x16(ld16(qoff[ks] + QB), ld16(kvb + ks * 1024), s);
      g = mfma_32x32x16(ld16(qoff[ks] + GB), ld16(kvb + L::KT + ks * 1024), g);
    }
    // register i holds query row 32qhalf + (i&7) + 8h + 16(i>>3) and key `key`
    const int qw0 = q0 + 32 * qhalf;  // first row of this wave's half
    const int bhq = b * a.Hq + hk * a.G + st / per_head;  // (batch, query head) of this step
    if (kw0 + 31 >= a.Nk || (a.causal && kw0 + 31 > qw0)) {
      // key past the end: every row masked; causal: rows before the key masked
      const int first_row = key >= a.Nk ? 0x7fffffff : (a.causal ? key : 0);
      const int thr = first_row == 0x7fffffff ? 64 : first_row - qw0 - 8 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (i & 7) + 16 * (i >> 3) < thr ? kNegInf : s[i];
    }
    // dropout: byte 2hi + (x >> 2) of kw[x & 3] is the random byte of row qw0 + 16hi + 8h + x
    // for this lane's key
    uint32_t kw[4] = {};
    if constexpr (DROP) drop_key_words(a.drop, (qw0 + 8 * h) >> 2, key, bhq, kw);
    // P = exp(scale S - L), dS = P (dP - D); the 8 rows (i&7) are consecutive, so L and D
    // come in as 16-byte LDS reads
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int lo = lb + BUF * BQ * 4 + 64 * hi;
      const f32x4 la = ld4f(lo), lbv = ld4f(lo + 16);
      const f32x4 da = ld4f(lo + 2 * BQ * 4), dbv = ld4f(lo + 2 * BQ * 4 + 16);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int i = 8 * hi + x;
        const float lv = x < 4 ? la[x] : lbv[x - 4], dvv = x < 4 ? da[x] : dbv[x - 4];
        const float p = fast_exp2(fmaf(s[i], a.c, -lv * kLog2e));
        if constexpr (DROP) {
          const bool z = drop_kept(a.drop, kw[x & 3], 2 * hi + (x >> 2));
          s[i] = keep_or_zero(z, p);  // P Z; dV takes 1 / (1 - p) at the end
          g[i] = p * fmaf(z ? g[i] : 0.f, a.drop.scale, -dvv);  // dS = P (dP Z / (1 - p) - D)
        } else {
          s[i] = p;                  // P
          g[i] = p * (g[i] - dvv);  // dS
        }
      }
    }
    // ---- dV += P^T dO, dK += dS^T Q over this wave's 32 rows (16 per product) ----
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int e = kk * 8;
      u32x4 pw, gw;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        pw[x] = pack_bf16x2(s[e + 2 * x], s[e + 2 * x + 1]);
        gw[x] = pack_bf16x2(g[e + 2 * x], g[e + 2 * x + 1]);
      }
      constexpr int R16 = 16 * L::ROW;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dv[db] = mfma_32x32x16(as_bf16x8(pw), tr8(troff[db][0] + GB + kk * R16, troff[db][1] + GB + kk * R16), dv[db]);
        dk[db] = mfma_32x32x16(as_bf16x8(gw), tr8(troff[db][0] + QB + kk * R16, troff[db][1] + QB + kk * R16), dk[db]);
      }
    }
  };

  issue_step(0);
  int st = 0;
  for (; st + 1 < n_steps; st += 2) {
    step(st, Const<0>{});
    step(st + 1, Const<1>{});
  }
  if (st < n_steps) step(st, Const<0>{});
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
    // Sum the halves in registers.
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dk[db][i] = (dk[db][i] + red[((2 * db) * 16 + i) * 64]) * a.scale;
        dv[db][i] += red[((2 * db + 1) * 16 + i) * 64];
        if constexpr (DROP) dv[db][i] *= a.drop.scale;
      }
    wave_sync();  // the fp32 reads above come before the bf16 tiles overwrite the area
    // Row-major bf16 tiles [32 keys][D] of dK and dV in this slice's area. Registers i, i+1
    // (i even) hold keys r, r+1 for dim 32db + l32; adjacent lanes swap one value so the even
    // lane packs dims (2m, 2m+1) of key r and the odd lane those of key r+1.
    constexpr int ROWB = D * 2;
    static_assert(2 * 32 * ROWB <= 2 * DB * 16 * 64 * 4, "bf16 tiles");
    char* tile = reinterpret_cast<char*>((float*)smem + (size_t)slice * (2 * DB * 16 * 64));
    const bool odd = lane & 1;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int row = 8 * (i >> 2) + 4 * h + (i & 3) + (odd ? 1 : 0);
        const int col = (32 * db + (l32 & ~1)) * 2;
        const float sk = __shfl_xor(odd ? dk[db][i] : dk[db][i + 1], 1);
        const float sv = __shfl_xor(odd ? dv[db][i] : dv[db][i + 1], 1);
        *(uint32_t*)(tile + row * ROWB + col) = odd ? pack_bf16x2(sk, dk[db][i + 1]) : pack_bf16x2(dk[db][i], sk);
        *(uint32_t*)(tile + 32 * ROWB + row * ROWB + col) =
            odd ? pack_bf16x2(sv, dv[db][i + 1]) : pack_bf16x2(dv[db][i], sv);
      }
    wave_sync();  // every lane's tile writes land before the lanes read each other's rows
    // 16-byte stores of whole row segments; rows past the end of the keys are dropped by the
    // buffer range.
    const long base = ((long)b * a.Nk + kw0) * a.k_row + hk * D;
    const long valid = kw0 < a.Nk ? ((long)(a.Nk - 1 - kw0) * a.k_row + D) * 2 : 0;
    const rsrc_t rdk = make_rsrc((uint16_t*)a.dk + base, valid);
    const rsrc_t rdv = make_rsrc((uint16_t*)a.dv + base, valid);
    constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
#pragma unroll
    for (int it = 0; it < 32 * CPR / 64; ++it) {
      const int c = it * 64 + lane, row = c / CPR, ch = c % CPR;
      const int goff = (int)(((long)row * a.k_row) * 2) + ch * 16;
      __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(tile + row * ROWB + ch * 16), rdk, goff, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(tile + 32 * ROWB + row * ROWB + ch * 16), rdv, goff, 0, 0);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Single-pass backward (d = 128, no dropout): the key-block-outer pass above also forms
// dQ += scale dS K for every tile, and the partial dQ of each 64-row query block is summed in
// fp32 by the key blocks one after another in a fixed order, so the sum is the same on every
// run (deterministic backward, "Flash Attention 3/4 笔记" (KaiSpace), causal scheduling part;
// dQ accumulated over key blocks as in Lecture 21 notes §2.6, exercise 6).
//
//  * Where the sums live: an fp32 copy of dQ in the workspace, one 4 KiB tile per (query head,
//    query block, wave), read with non-temporal loads (they do not hit the compute unit's L1)
//    and written with plain stores (the L1 writes through), so the XCD's L2 is the point of
//    coherence. All key blocks of a (batch, kv head) therefore run on one XCD: workgroups take
//    tasks from a per-XCD pool (hardware register XCC_ID), heads assigned to pools round-robin.
//  * Order without a separate counter: the low 8 bits of every fp32 partial sum hold how many
//    key blocks have added to it (the sum is kept to a 15-bit significand, rounded to nearest;
//    far finer than the bf16 result). The key block of rank r (0 = first) waits until every value
//    it loaded carries tag r, adds its part and stores the values with tag r + 1; the last one
//    writes dQ in bf16 and stores zeros, so the area is all zero between calls. A value is read
//    only once its writer has stored it, and a writer never waits for a reader, so a wait chain
//    always ends at a block's first adder.
//  * Visiting order. Causal: key block j sees query blocks i >= 2j and walks them downwards from
//    the last, the G heads of the group at each block, adding in order of decreasing j (tasks
//    are taken shortest first). Every key block reaches a block the same number of steps after
//    its own start, so j arrives after j + 1, which was taken before it, and a block's adders
//    follow one another at the pace tasks are taken: its partial sum and Q/dO tiles are live
//    for a few steps rather than from the first adder's visit to key block 0's, and fewer
//    blocks are live at once than the L2 holds. The first writer of a block never waits.
//    Without the mask: every key block walks all M = G Tr blocks of the group in the same
//    order, and tasks are taken in decreasing j too, so key block j follows j + 1 through the
//    blocks a fraction of a step behind it (a convoy that forms once, at the start). An order
//    with one adder per block per step needs a circular order of the adders, and so all Tc
//    workgroups of a head running together, which two calls on two streams can prevent.
//  * Pools are taken in order and a task only waits for a task of its own head taken before
//    it, so the waits end with any number of workgroups resident; each wait is also bounded: a
//    wave whose wait outlasts 0.2 s (possible only if the area was not zero at the start) stops
//    waiting for the rest of the launch, the result is then wrong, and the event is counted in a
//    word of the workspace that the kernel never clears, so a caller checking that the counters
//    are zero after a call sees it.
//  * Per step, after the dK/dV products: each wave writes its dS^T (32 keys x 32 rows, bf16) to
//    LDS; after a barrier each wave computes dQ^T for its 32 rows x 32 dims of the 64 x 128 block
//    over all 128 keys, K^T and dS^T both read transposed with ds_read_b64_tr_b16. K and V keep
//    the fragment order of the score products, with the 16-byte slots permuted so the transposed
//    K^T reads are free of bank conflicts too.
// D = rowsum(dO * O) comes from a small kernel that runs first.
constexpr int kMaxPools = 8;          // task pools: one per XCD (a.ctr[0..7]; a.ctr[8] counts leavers)
constexpr int kTimeoutCounter = kBwdPoolCounters - 1;  // waits that ran out (left nonzero)
static_assert(kMaxPools + 1 < kTimeoutCounter, "pool counters");
constexpr int kCusPerXcd = 32;
constexpr int kMaxAdders = 255;       // 8-bit adder tags
constexpr long kWaitTicks = 20000000;  // bounded waits: 0.2 s of the 100 MHz real-time counter

template <int D>
struct FusedLds {
  using B = BwdLds<D>;
  static constexpr int OFF_DS = B::BYTES;              // dS^T [128 keys][64 rows] bf16, swizzled
  static constexpr int DS_BYTES = BK * BQ * 2;
  static constexpr int BYTES = OFF_DS + DS_BYTES;
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// 16-byte slot of fragment lane l in 1 KiB region r of a K/V block (an involution).
__device__ __forceinline__ int frag_slot(int l, int r) { return l ^ (4 * (l >> 5)) ^ (8 * (r & 1)); }

// 16-byte chunk swizzle of the dS^T rows (128 bytes per key): conflict-free for the 16-byte
// writes (16 consecutive keys, one chunk) and for the transposed reads (4 keys x 2 chunks).
__device__ __forceinline__ int ds_swz(int key) { return (((key >> 1) & 1) << 2) | ((key >> 2) & 3); }

// dma_frag with the slot permutation: slot s of region r holds fragment lane frag_slot(s, r).
template <int D, int NLOAD>
__device__ __forceinline__ void dma_frag_p(char* dst, const uint16_t* src, long row_stride, int valid_rows) {
  constexpr int KS = D / 16;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const u32x4 r = dma_rsrc(src, ((long)(valid_rows - 1) * row_stride + D) * 2);
#pragma unroll
  for (int p = 0; p < NLOAD; ++p) {
    const int region = kWaves * p + w;
    const int l = frag_slot(lane, region);
    const int row = 32 * (region / KS) + (l & 31);
    const int voff = (int)((row * row_stride + 16 * (region % KS) + 8 * (l >> 5)) * 2);
    lds_dma16(r, dst + region * 1024, voff);
  }
}

// LDS-only barrier: this wave's LDS accesses are done, then the workgroup barrier (vector memory
// operations may stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// v ^ c in a VALU instruction the compiler keeps where it is written (not hoisted out of the
// loop into a register of its own).
__device__ __forceinline__ int xor_imm(int v, int c) {
  int r;
  asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "i"(c), "v"(v));
  return r;
}

// One wave's 4 KiB partial-sum tile: lane l holds values 4 r4 .. 4 r4 + 3 at byte (64 r4 + l) 16.
__device__ __forceinline__ void load_tile(const rsrc_t& r, int lane, f32x16& x) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (r4 * 64 + lane) * 16, 0, 2));
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * r4 + e] = v[e];
  }
}
__device__ __forceinline__ void store_tile(const rsrc_t& r, int lane, const f32x16& x) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x[4 * r4 + e];
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (r4 * 64 + lane) * 16, 0, 0);
  }
}
// Whether any value of the wave's tile carries a tag other than `tag`. (__float_as_uint on each
// element: __builtin_bit_cast applied to a vector element is lowered as a cast of element 0.)
__device__ __forceinline__ bool tile_stale(const f32x16& x, int tag) {
  uint32_t diff = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) diff |= __float_as_uint(x[e]) ^ (uint32_t)tag;
  return __builtin_amdgcn_ballot_w64((diff & 0xffu) != 0) != 0;
}
// fp32 sum -> 15-bit significand rounded to nearest (ties away from zero), tag in the low 8 bits.
__device__ __forceinline__ float tag_value(float v, int tag) {
  return __builtin_bit_cast(float, ((__builtin_bit_cast(uint32_t, v) + 0x80u) & ~0xffu) | (uint32_t)tag);
}
__device__ __forceinline__ float untag(float v) { return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & ~0xffu); }

// D[b, h, n] = rowsum(dO * O) over the head dimension; 16 lanes per row, rows in memory order.
template <int D>
__global__ __launch_bounds__(256) void bwd_dvec_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row (16 bytes each)
  const long n_rows = (long)a.B * a.Nq * a.Hq;
  const int sub = threadIdx.x % LPR;
  for (long row = ((long)blockIdx.x * blockDim.x + threadIdx.x) / LPR; row < n_rows;
       row += (long)gridDim.x * blockDim.x / LPR) {
    const long off = row * D + sub * 8;  // Q-layout rows are contiguous: [B, Nq, Hq, D]
    const u32x4 ow = *(const u32x4*)((const uint16_t*)a.o + off);
    const u32x4 gw = *(const u32x4*)((const uint16_t*)a.dout + off);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(bf16_lo(ow[e]), bf16_lo(gw[e]), s);
      s = fmaf(bf16_hi(ow[e]), bf16_hi(gw[e]), s);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (sub == 0) {
      const int hq = (int)(row % a.Hq);
      const long bn = row / a.Hq;
      const int n = (int)(bn % a.Nq), b = (int)(bn / a.Nq);
      a.dvec[((long)b * a.Hq + hq) * a.Nq + n] = s;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kMainThreads, 1) void bwd_fused_kernel(BwdArgs a) {
  using L = BwdLds<D>;
  using F = FusedLds<D>;
  constexpr int KS = D / 16, DB = D / 32;
  static_assert(D == 128, "one 32-dim slice of dQ per key-slice wave");
  static_assert(L::STEP_DMA < 60, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[F::BYTES];
  __shared__ int s_task;
  char* kl = smem + L::OFF_K;
  char* vl = smem + L::OFF_V;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int slice = wave & 3;   // 32-key slice of the block; also this wave's 32 dims of dQ
  const int qhalf = wave >> 2;  // 32-row half of each 64-row query block

  const int n_tr = (a.Nq + BQ - 1) / BQ;  // query blocks per head
  const int n_tc = a.n_kvblk;             // key blocks per head
  const int pool = xcc_id() % a.n_pools;
  const int n_heads = a.B * a.Hkv;
  const int pool_heads = pool < n_heads ? (n_heads - pool + a.n_pools - 1) / a.n_pools : 0;
  const int pool_tasks = pool_heads * n_tc;

  // ---- per-lane LDS offsets, fixed for the kernel ----
  // The swizzled offsets of the Q / dO row reads (16-dim step ks) and of the transposed dO / Q
  // reads (32-dim slice db) differ from one base by an XOR with ks << 5 and db << 6 (the
  // swizzle only moves those bits); the XOR is done at each use to save registers.
  int q_base, tr_base[2];
  {
    const int row = 32 * qhalf + swap_bits23(l32);
    q_base = row * L::ROW + ((h ^ t_swz<D>(row)) << 4);
    const int sl = lane & 15, g = lane >> 4;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int rr = 8 * (g >> 1) + 4 * rd + (sl >> 2);
      const int col_b = (16 * (g & 1) + 4 * (sl & 3)) * 2;
      tr_base[rd] = (32 * qhalf + rr) * L::ROW + (((col_b >> 4) ^ t_swz<D>(rr)) << 4) + (col_b & 15);
    }
  }
  auto qoff = [&](int ks) { return xor_imm(q_base, ks << 5); };
  auto troff = [&](int db, int rd) { return xor_imm(tr_base[rd], db << 6); };
  // K / V fragments of the score products (slot permuted by region parity = ks parity)
  const int kvb0 = L::OFF_K + slice * KS * 1024 + 16 * frag_slot(lane, 0);
  const int kvb1 = L::OFF_K + slice * KS * 1024 + 16 * frag_slot(lane, 1);
  // K^T as the A operand of dQ^T (A row m = dim 32 slice + swap_bits23(m), so accumulator
  // register i holds dim 32 slice + (i&7) + 8h + 16(i>>3)); 16-key step kk adds 8192 (kk>>1) +
  // 256 (kk&1). Source lane s of 16-lane group g reads key 8(g>>1) + 4rd + s/4 and the 4 dims
  // that the transpose hands to lanes 4(s%4) .. +3.
  int kt_off[2], ds_off[2];
  {
    const int s = lane & 15, g = lane >> 4, q = s & 3;
    const int sw = ((q & 1) << 1) | (q >> 1), hh = sw >> 1, ll = sw & 1;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      kt_off[rd] = L::OFF_K + 1024 * (2 * slice + (g & 1)) +
                   16 * (8 * ((g >> 1) ^ (g & 1)) + 4 * (rd ^ hh) + (s >> 2) + 32 * hh) + 8 * ll;
      // dS^T as the B operand: key 8(g>>1) + 4rd + s/4 (+16 kk: 2048 bytes), rows
      // 32 qhalf + 16(g&1) + 4(s%4) .. +3
      const int key = 8 * (g >> 1) + 4 * rd + (s >> 2);
      const int c = 4 * qhalf + 2 * (g & 1) + (q >> 1);
      ds_off[rd] = F::OFF_DS + key * 128 + 16 * (c ^ ds_swz(key)) + 8 * (s & 1);
    }
  }
  const int lb = L::OFF_L + (32 * qhalf + 8 * h) * 4;
  auto ld16 = [&](int off) { return *(const bf16x8*)(smem + off); };
  auto ld4f = [&](int off) { return *(const f32x4*)(smem + off); };
  auto tr8 = [&](int off0, int off1) {
    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + off0));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + off1));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  bool gave_up = false;  // a bounded wait of this wave ran out: wait no more in this launch
  for (;;) {
    // every wave is done with the previous task's LDS and memory operations
    wait_vm_barrier<0>();
    if (t == 0) s_task = __hip_atomic_fetch_add(a.ctr + pool, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vm_barrier<0>();
    const int task = __builtin_amdgcn_readfirstlane(s_task);
    if (task >= pool_tasks) break;
    const int bhk = pool + a.n_pools * (task / n_tc);
    const int jj = task % n_tc;
    const int j = n_tc - 1 - jj;  // decreasing j: with the mask the shortest task first
    const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
    const int kv0 = j * BK;
    const int kw0 = kv0 + slice * 32;
    const int key = kw0 + l32;
    const uint16_t* kp = (const uint16_t*)a.k + (long)b * a.Nk * a.k_row + hk * D;
    const uint16_t* vp = (const uint16_t*)a.v + (long)b * a.Nk * a.k_row + hk * D;
    dma_frag_p<D, L::KDMA>(kl, kp + (long)kv0 * a.k_row, a.k_row, a.Nk - kv0);
    dma_frag_p<D, L::KDMA>(vl, vp + (long)kv0 * a.k_row, a.k_row, a.Nk - kv0);

    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

    const int qb_first = a.causal ? kv0 / BQ : 0;
    const int per_head = n_tr - qb_first;
    const int n_steps = a.G * per_head;
    const int bhq0 = b * a.Hq + hk * a.G;

    // A step's visit packed in one word: bits 0-7 this key block's rank among the adders of the
    // block (0 = first), bit 8 whether it is the last, bits 9-15 the query head g within the
    // group, bits 16-31 the 64-row block i. The walk state (sa, sb) is (g, i) with the mask and
    // (unused, g Tr + i) without.
    auto make_vis = [&](int sa, int sb) {
      int g, i, rank;
      bool last;
      if (a.causal) {
        g = sa;
        i = sb;
        const int cnt = min(n_tc, (BQ * i + BQ - 1) / BK + 1);  // key blocks 0 .. cnt-1 add
        rank = cnt - 1 - j;
        last = j == 0;
      } else {
        g = sb / n_tr;
        i = sb - g * n_tr;
        rank = n_tc - 1 - j;
        last = j == 0;
      }
      return rank | (last ? 256 : 0) | (g << 9) | (i << 16);
    };
    auto advance = [&](int& sa, int& sb) {
      if (a.causal) {
        if (++sa == a.G) {
          sa = 0;
          --sb;
        }
        // uniform, so that the tile addresses built from them stay in scalar registers
        sa = __builtin_amdgcn_readfirstlane(sa);
        sb = __builtin_amdgcn_readfirstlane(sb);
      } else {
        ++sb;
      }
    };
    auto vis_g = [](int v) { return (v >> 9) & 127; };
    auto vis_i = [](int v) { return (int)((unsigned)v >> 16); };
    auto vis_rank = [](int v) { return v & 255; };
    int sa = 0, sb = a.causal ? n_tr - 1 : 0;
    int cur = make_vis(sa, sb);
    auto tile_index = [&](int v) {  // (query head, block, wave) tile of dQ
      return ((bhq0 + vis_g(v)) * n_tr + vis_i(v)) * kWaves + wave;
    };

    auto issue_step = [&](int v, int buf) {
      const int hq = hk * a.G + vis_g(v), q0 = vis_i(v) * BQ;
      const long qo = ((long)b * a.Nq + q0) * a.q_row + hq * D;
      dma_rows<D, L::QDMA>(smem + L::OFF_Q + buf * L::QT, (const uint16_t*)a.q + qo, a.q_row, a.Nq - q0);
      dma_rows<D, L::QDMA>(smem + L::OFF_DO + buf * L::QT, (const uint16_t*)a.dout + qo, a.q_row, a.Nq - q0);
      const long loff = ((long)b * a.Hq + hq) * a.Nq + q0;
      const long lbytes = (long)min(BQ, a.Nq - q0) * 4;
      if (qhalf == 0) lds_dma4(dma_rsrc(a.lse + loff, lbytes), smem + L::OFF_L + buf * BQ * 4, lane * 4);
      else lds_dma4(dma_rsrc(a.dvec + loff, lbytes), smem + L::OFF_D + buf * BQ * 4, lane * 4);
    };

    bool prev_last = false;  // the previous step stored dQ (eight stores instead of four)

    auto step = [&](const int st, auto bufc) {
      constexpr int BUF = decltype(bufc)::value;
      constexpr int QB = L::OFF_Q + BUF * L::QT, GB = L::OFF_DO + BUF * L::QT;
      const int g = vis_g(cur), q0 = vis_i(cur) * BQ, rank = vis_rank(cur);
      const bool last = (cur >> 8) & 1;
      const int tile = tile_index(cur);
      // this step's loads have landed and every wave is done with the previous step's LDS (the
      // previous step's dQ stores, its last vector-memory operations, may still be in flight)
      if (st == 0) wait_vm_barrier<0>();
      else if (prev_last) wait_vm_barrier<8>();
      else wait_vm_barrier<4>();
      int nxt = cur;
      if (st + 1 < n_steps) {
        advance(sa, sb);
        nxt = make_vis(sa, sb);
        issue_step(nxt, BUF ^ 1);
      }
      const rsrc_t racc = make_rsrc(a.dq_acc + (long)tile * 1024, 4096);

      // ---- S = Q K^T and dP = dO V^T for this wave's 32 rows x 32 keys ----
      f32x16 s, gg;
      zero16(s);
      zero16(gg);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int kb = (ks & 1 ? kvb1 : kvb0) + ks * 1024;
        const int qo = qoff(ks);
        s = mfma_32x32x16(ld16(qo + QB), ld16(kb), s);
        gg = mfma_32x32x16(ld16(qo + GB), ld16(kb + L::KT), gg);
      }
      // the partial sum of this tile, stored by the previous adder at the end of its step
      f32x16 dq;
      if (rank != 0) load_tile(racc, lane, dq);
      else zero16(dq);
      const int qw0 = q0 + 32 * qhalf;
      if (kw0 + 31 >= a.Nk || (a.causal && kw0 + 31 > qw0)) {
        const int first_row = key >= a.Nk ? 0x7fffffff : (a.causal ? key : 0);
        const int thr = first_row == 0x7fffffff ? 64 : first_row - qw0 - 8 * h;
#pragma unroll
        for (int x = 0; x < 16; ++x) s[x] = (x & 7) + 16 * (x >> 3) < thr ? kNegInf : s[x];
      }
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int lo = lb + BUF * BQ * 4 + 64 * hi;
        const f32x4 la = ld4f(lo), lbv = ld4f(lo + 16);
        const f32x4 da = ld4f(lo + 2 * BQ * 4), dbv = ld4f(lo + 2 * BQ * 4 + 16);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int r = 8 * hi + x;
          const float lv = x < 4 ? la[x] : lbv[x - 4], dvv = x < 4 ? da[x] : dbv[x - 4];
          const float p = fast_exp2(fmaf(s[r], a.c, -lv * kLog2e));
          s[r] = p;                   // P
          gg[r] = p * (gg[r] - dvv);  // dS
        }
      }
      // ---- dV += P^T dO, dK += dS^T Q; dS^T (bf16) to LDS for the dQ product ----
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int e = kk * 8;
        u32x4 pw, gw;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          pw[x] = pack_bf16x2(s[e + 2 * x], s[e + 2 * x + 1]);
          gw[x] = pack_bf16x2(gg[e + 2 * x], gg[e + 2 * x + 1]);
        }
        {
          const int kyb = 32 * slice + l32;
          const int c = 4 * qhalf + 2 * kk + h;
          *(u32x4*)(smem + F::OFF_DS + kyb * 128 + 16 * (c ^ ds_swz(kyb))) = gw;
        }
        constexpr int R16 = 16 * L::ROW;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int t0 = troff(db, 0), t1 = troff(db, 1);
          dv[db] = mfma_32x32x16(as_bf16x8(pw), tr8(t0 + GB + kk * R16, t1 + GB + kk * R16), dv[db]);
          dk[db] = mfma_32x32x16(as_bf16x8(gw), tr8(t0 + QB + kk * R16, t1 + QB + kk * R16), dk[db]);
        }
      }
      lds_barrier();  // every wave's dS^T is in LDS

      // ---- wait until every value of the tile carries this key block's rank ----
      if (rank != 0) {
        if (tile_stale(dq, rank) && !gave_up) {
          const unsigned long long t_start = __builtin_amdgcn_s_memrealtime();
          do {
            __builtin_amdgcn_s_sleep(2);
            asm volatile("" ::: "memory");
            load_tile(racc, lane, dq);
            if (__builtin_amdgcn_s_memrealtime() - t_start > (unsigned long long)kWaitTicks) gave_up = true;
          } while (tile_stale(dq, rank) && !gave_up);
          // count a wait that ran out where the caller can see it (never reset by the kernel)
          if (gave_up && lane == 0)
            __hip_atomic_fetch_add(a.ctr + kTimeoutCounter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[e] = untag(dq[e]);
      }

      // ---- dQ^T (this wave's 32 dims x 32 rows) += K^T dS^T over the block's 128 keys ----
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int ko = 8192 * (kk >> 1) + 256 * (kk & 1);
        dq = mfma_32x32x16(tr8(kt_off[0] + ko, kt_off[1] + ko), tr8(ds_off[0] + 2048 * kk, ds_off[1] + 2048 * kk), dq);
      }
      if (last) {
        // dQ = scale * sum, bf16: row q0 + 32 qhalf + l32, dims 32 slice + 16 hi + 8h + 4 qq .. +3;
        // then the tile back to zero for the next call
        const int hq = hk * a.G + g;
        const long qbase = (long)b * a.Nq * a.q_row + hq * D;
        const rsrc_t rdq = make_rsrc((uint16_t*)a.dq + qbase, ((long)(a.Nq - 1) * a.q_row + D) * 2);
        const int row = q0 + 32 * qhalf + l32;
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int r0 = 8 * hi + 4 * qq;
            u32x2 w;
            w[0] = pack_bf16x2(dq[r0] * a.scale, dq[r0 + 1] * a.scale);
            w[1] = pack_bf16x2(dq[r0 + 2] * a.scale, dq[r0 + 3] * a.scale);
            __builtin_amdgcn_raw_buffer_store_b64(w, rdq, (int)(((long)row * a.q_row + 32 * slice + 16 * hi + 8 * h + 4 * qq) * 2), 0, 0);
          }
        f32x16 z;
        zero16(z);
        store_tile(racc, lane, z);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[e] = tag_value(dq[e], rank + 1);
        store_tile(racc, lane, dq);
      }
      prev_last = last;
      cur = nxt;
    };

    issue_step(cur, 0);
    int st = 0;
    for (; st + 1 < n_steps; st += 2) {
      step(st, Const<0>{});
      step(st + 1, Const<1>{});
    }
    if (st < n_steps) step(st, Const<0>{});
    __builtin_amdgcn_s_waitcnt(0);

    // ---- dK/dV epilogue, as in the two-kernel path ----
    wait_vm_barrier<0>();
    float* red = (float*)smem + (size_t)slice * (2 * DB * 16 * 64) + lane;
    if (qhalf == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          red[((2 * db) * 16 + x) * 64] = dk[db][x];
          red[((2 * db + 1) * 16 + x) * 64] = dv[db][x];
        }
    }
    wait_vm_barrier<0>();
    if (qhalf == 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          dk[db][x] = (dk[db][x] + red[((2 * db) * 16 + x) * 64]) * a.scale;
          dv[db][x] += red[((2 * db + 1) * 16 + x) * 64];
        }
      wave_sync();
      constexpr int ROWB = D * 2;
      char* tl = reinterpret_cast<char*>((float*)smem + (size_t)slice * (2 * DB * 16 * 64));
      const bool odd = lane & 1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; x += 2) {
          const int row = 8 * (x >> 2) + 4 * h + (x & 3) + (odd ? 1 : 0);
          const int col = (32 * db + (l32 & ~1)) * 2;
          const float sk = __shfl_xor(odd ? dk[db][x] : dk[db][x + 1], 1);
          const float sv = __shfl_xor(odd ? dv[db][x] : dv[db][x + 1], 1);
          *(uint32_t*)(tl + row * ROWB + col) = odd ? pack_bf16x2(sk, dk[db][x + 1]) : pack_bf16x2(dk[db][x], sk);
          *(uint32_t*)(tl + 32 * ROWB + row * ROWB + col) =
              odd ? pack_bf16x2(sv, dv[db][x + 1]) : pack_bf16x2(dv[db][x], sv);
        }
      wave_sync();
      const long base = ((long)b * a.Nk + kw0) * a.k_row + hk * D;
      const long valid = kw0 < a.Nk ? ((long)(a.Nk - 1 - kw0) * a.k_row + D) * 2 : 0;
      const rsrc_t rdk = make_rsrc((uint16_t*)a.dk + base, valid);
      const rsrc_t rdv = make_rsrc((uint16_t*)a.dv + base, valid);
      constexpr int CPR = ROWB / 16;
#pragma unroll
      for (int it = 0; it < 32 * CPR / 64; ++it) {
        const int c = it * 64 + lane, row = c / CPR, ch = c % CPR;
        const int goff = (int)(((long)row * a.k_row) * 2) + ch * 16;
        __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(tl + row * ROWB + ch * 16), rdk, goff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(tl + 32 * ROWB + row * ROWB + ch * 16), rdv, goff, 0, 0);
      }
    }
  }
  // the last workgroup to leave resets the pool counters for the next call
  if (t == 0) {
    const int fin = __hip_atomic_fetch_add(a.ctr + kMaxPools, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (fin == (int)gridDim.x - 1) {
      for (int p = 0; p <= kMaxPools; ++p) __hip_atomic_store(a.ctr + p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------------------------------
// dQ = scale * dS K, query-block outer (no atomics): each wave owns 32 query rows and keeps
// Q, dO, L and D of its rows in registers while 64-key K/V tiles stream through a four-buffer
// LDS ring (direct-to-LDS loads three tiles ahead). Per tile, as in the forward, the products
// come out transposed with one query per lane: S^T = K Q^T and dP^T = V dO^T (K and V rows
// relabelled so each lane half holds 8 consecutive keys), then P = exp(scale*S - L) and
// dS = P * (dP - D) are per-lane scalar work, and dS^T goes from the accumulator straight into
// the B operand of dQ^T += K^T dS^T, K^T read transposed from the same K tile.
constexpr int DQ_BR = kBwdDqRows;  // 256 query rows per workgroup
constexpr int DQ_BC = kBwdDqKeys;  // 64 keys per tile
constexpr int DQ_NBUF = 4;

template <int D>
struct DqTile {
  static constexpr int ROW = D * 2;
  static constexpr int T_BYTES = DQ_BC * ROW;              // K or V tile
  static constexpr int BUF = 2 * T_BYTES;                  // K then V
  static constexpr int RR = 1024 / ROW;                    // rows per 1 KiB load
  static constexpr int DMA = T_BYTES / 1024 / kWaves;      // loads per wave per tensor per tile
  static constexpr int VMCNT = 2 * DMA;                    // loads per wave per tile
};

// This wave's share of the direct-to-LDS loads of the K and V tile starting at key kv0.
template <int D>
__device__ __forceinline__ void dq_dma_tile(char* buf, const uint16_t* kp, const uint16_t* vp, long k_row, int kv0,
                                            int nk) {
  using T = DqTile<D>;
  dma_rows<D, T::DMA>(buf, kp + (long)kv0 * k_row, k_row, nk - kv0);
  dma_rows<D, T::DMA>(buf + T::T_BYTES, vp + (long)kv0 * k_row, k_row, nk - kv0);
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kMainThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using T = DqTile<D>;
  constexpr int KS = D / 16, DB = D / 32;
  static_assert(3 * T::VMCNT < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) char smem[DQ_NBUF * T::BUF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  int bh, qb;
  if (CAUSAL) {  // longest first, each XCD keeping its own heads
    int lvl;
    xcd_longest_first((int)blockIdx.x, a.n_tasks_dq / a.n_qblk_dq, a.n_qblk_dq, bh, lvl);
    qb = a.n_qblk_dq - 1 - lvl;
  } else {
    const int task = xcd_contiguous_task(blockIdx.x, a.n_tasks_dq);
    bh = task / a.n_qblk_dq;
    qb = task % a.n_qblk_dq;
  }
  const int b = bh / a.Hq, hq = bh % a.Hq, hk = hq / a.G;
  const long qbase = (long)b * a.Nq * a.q_row + hq * D;
  const uint16_t* kp = (const uint16_t*)a.k + (long)b * a.Nk * a.k_row + hk * D;
  const uint16_t* vp = (const uint16_t*)a.v + (long)b * a.Nk * a.k_row + hk * D;
  const long q_valid = ((long)(a.Nq - 1) * a.q_row + D) * 2;

  // rows interleaved over the waves so a causal block's work is even across them
  const int q0 = qb * DQ_BR + 32 * wave;
  const int qi = q0 + l32;  // this lane's query row
  // Q and dO as B operands of S^T = K Q^T and dP^T = V dO^T: column qi, dims [16ks + 8h, +8)
  bf16x8 qf[KS], gf[KS];
  // D = rowsum(dO * O) of row qi (§2.6), from this lane's half of the dims and its partner's;
  // written for the dK/dV kernel, which runs after this one (rows past Nq read zeros)
  float dd = 0.f;
  {
    const rsrc_t rq = make_rsrc((const uint16_t*)a.q + qbase, q_valid);
    const rsrc_t rg = make_rsrc((const uint16_t*)a.dout + qbase, q_valid);
    const rsrc_t ro = make_rsrc((const uint16_t*)a.o + qbase, q_valid);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = (int)(((long)qi * a.q_row + ks * 16 + h * 8) * 2);
      qf[ks] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      const u32x4 gw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
      const u32x4 ow = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
      gf[ks] = as_bf16x8(gw);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dd = fmaf(bf16_lo(ow[e]), bf16_lo(gw[e]), dd);
        dd = fmaf(bf16_hi(ow[e]), bf16_hi(gw[e]), dd);
      }
    }
  }
  dd = halves_sum(dd);
  float l2 = 0.f;  // L in base 2 of row qi (rows past Nq contribute nothing)
  if (qi < a.Nq) {
    l2 = a.lse[((long)b * a.Hq + hq) * a.Nq + qi] * kLog2e;
    if (h == 0) a.dvec[((long)b * a.Hq + hq) * a.Nq + qi] = dd;
  }

  int n_tiles = (a.Nk + DQ_BC - 1) / DQ_BC;
  int last_w = n_tiles - 1;
  if (CAUSAL) {
    n_tiles = min(n_tiles, (min(a.Nq, (qb + 1) * DQ_BR) - 1) / DQ_BC + 1);
    last_w = min(n_tiles - 1, (q0 + 31) / DQ_BC);
  }
  const int nk_load = min(a.Nk, n_tiles * DQ_BC);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) zero16(acc[db]);

  // the compiler does not count the asm loads below: its own loads complete first
  __builtin_amdgcn_s_waitcnt(0);
  dq_dma_tile<D>(smem, kp, vp, a.k_row, 0, nk_load);
  dq_dma_tile<D>(smem + T::BUF, kp, vp, a.k_row, DQ_BC, nk_load);
  dq_dma_tile<D>(smem + 2 * T::BUF, kp, vp, a.k_row, 2 * DQ_BC, nk_load);

  // Per-lane LDS byte offsets within a tile buffer, fixed for the whole task; the buffer,
  // tensor and step parts of each address are constants in the instructions' offset field.
  // K / V rows as A operands of S^T and dP^T: row 32 kb + relabelled l32, logical chunk 2 ks + h.
  int roff[2][KS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * kb + swap_bits23(l32);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[kb][ks] = row * T::ROW + (((2 * ks + h) ^ t_swz<D>(row)) << 4);
  }
  // K^T as the A operand of dQ^T (two ds_read_b64_tr_b16 per fragment, as in the dK/dV kernel)
  int troff[DB][2];
  {
    const int sl = lane & 15, g = lane >> 4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int rr = 8 * (g >> 1) + 4 * rd + (sl >> 2);
        const int col_b = (32 * db + 16 * (g & 1) + 4 * (sl & 3)) * 2;
        troff[db][rd] = rr * T::ROW + (((col_b >> 4) ^ t_swz<D>(rr)) << 4) + (col_b & 15);
      }
  }
  auto ld16 = [&](int off) { return *(const bf16x8*)(smem + off); };
  auto tr8 = [&](int off0, int off1) {
    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + off0));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + off1));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // One tile; the buffer index j % DQ_NBUF is a compile-time constant in each copy.
  auto tile = [&](const int j, auto bufc) {
    constexpr int KB = decltype(bufc)::value * T::BUF, VB = KB + T::T_BYTES;
    // tile j landed (tiles j+1 and j+2 may be pending); every wave is done with tile j-1,
    // whose buffer the prefetch of tile j+3 refills
    wait_vm_barrier<2 * T::VMCNT>();
    dq_dma_tile<D>(smem + ((j + 3) % DQ_NBUF) * T::BUF, kp, vp, a.k_row, (j + 3) * DQ_BC, nk_load);
    if (j > last_w) return;
    const int kv0 = j * DQ_BC;

    // ---- S^T and dP^T for 64 keys (two 32-key blocks) x this wave's 32 queries ----
    f32x16 s[2], g[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      zero16(s[kb]);
      zero16(g[kb]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s[kb] = mfma_32x32x16(ld16(roff[kb][ks] + KB), qf[ks], s[kb]);
        g[kb] = mfma_32x32x16(ld16(roff[kb][ks] + VB), gf[ks], g[kb]);
      }
      fence();  // bounds the K/V fragments in flight (register budget)
    }
    // register i of block kb holds key kv0 + 32kb + (i&7) + 8h + 16(i>>3), query qi
    if (kv0 + DQ_BC > a.Nk || (CAUSAL && kv0 + DQ_BC - 1 > q0)) {
      // keys at or past min(Nk, qi + 1 when causal) are masked
      const int thr = (CAUSAL ? min(a.Nk, qi + 1) : a.Nk) - kv0 - 8 * h;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 32 * kb + (i & 7) + 16 * (i >> 3) >= thr ? kNegInf : s[kb][i];
    }
    // dropout: byte x & 3 of kw[4kb + 2hi + (x >> 2)] is the random byte of key
    // kv0 + 32kb + 16hi + 8h + x for row qi
    uint32_t kw[8] = {};
    if constexpr (DROP) drop_row_words(a.drop, (kv0 + 8 * h) >> 2, qi, bh, kw);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int i = 8 * hi + x;
          const float p = fast_exp2(fmaf(s[kb][i], a.c, -l2));
          if constexpr (DROP) {  // dS = P (dP Z / (1 - p) - D)
            const bool z = drop_kept(a.drop, kw[4 * kb + 2 * hi + (x >> 2)], x & 3);
            g[kb][i] = p * fmaf(z ? g[kb][i] : 0.f, a.drop.scale, -dd);
          } else {
            g[kb][i] = p * (g[kb][i] - dd);  // dS
          }
        }
      }
    // ---- dQ^T += K^T dS^T: 16-key step kk takes dS registers 8(kk&1) .. +7 of block kk/2 ----
#pragma unroll
    for (int kk = 0; kk < DQ_BC / 16; ++kk) {
      const f32x16& gs = g[kk >> 1];
      const int e = (kk & 1) * 8;
      u32x4 gw;
#pragma unroll
      for (int x = 0; x < 4; ++x) gw[x] = pack_bf16x2(gs[e + 2 * x], gs[e + 2 * x + 1]);
      constexpr int R16 = 16 * T::ROW;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc[db] = mfma_32x32x16(tr8(troff[db][0] + KB + kk * R16, troff[db][1] + KB + kk * R16), as_bf16x8(gw),
                                acc[db]);
    }
  };
  // unrolled by the ring size; the iteration count is padded to a multiple of it (the extra
  // iterations only keep the barrier count and prefetch nothing)
  static_assert(DQ_NBUF == 4, "one tile copy per buffer");
  for (int j = 0; j < n_tiles; j += 4) {
    tile(j, Const<0>{});
    tile(j + 1, Const<1>{});
    tile(j + 2, Const<2>{});
    tile(j + 3, Const<3>{});
  }
  __builtin_amdgcn_s_waitcnt(0);  // drain the tail prefetches before the workgroup ends

  // ---- dQ = scale * acc (bf16); register i of acc[db] is dim 32db + 8(i/4) + 4h + i%4 ----
  const rsrc_t rdq = make_rsrc((uint16_t*)a.dq + qbase, q_valid);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 w;
      w[0] = pack_bf16x2(acc[db][4 * jj + 0] * a.scale, acc[db][4 * jj + 1] * a.scale);
      w[1] = pack_bf16x2(acc[db][4 * jj + 2] * a.scale, acc[db][4 * jj + 3] * a.scale);
      __builtin_amdgcn_raw_buffer_store_b64(w, rdq, (int)(((long)qi * a.q_row + 32 * db + 8 * jj + 4 * h) * 2), 0, 0);
    }
}

// The dQ kernel runs first: besides dQ it computes D = rowsum(dO * O) for its rows (every row
// belongs to exactly one of its workgroups) and stores it for the dK/dV kernel.
template <int D, bool DROP>
hipError_t launch_two_pass(const BwdArgs& a, hipStream_t s) {
  if (a.causal) hipLaunchKernelGGL((bwd_dq_kernel<D, true, DROP>), dim3(a.n_tasks_dq), dim3(kMainThreads), 0, s, a);
  else hipLaunchKernelGGL((bwd_dq_kernel<D, false, DROP>), dim3(a.n_tasks_dq), dim3(kMainThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_main_kernel<D, DROP>), dim3(a.n_tasks), dim3(kMainThreads), 0, s, a);
  return hipGetLastError();
}

// Single pass: D first, then the persistent key-block-outer kernel, one workgroup per compute
// unit.
hipError_t launch_single_pass(BwdArgs a, hipStream_t s) {
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  a.n_pools = max(1, min(kMaxPools, n_cu / kCusPerXcd));
  const long rows = (long)a.B * a.Nq * a.Hq;
  const long dwant = (rows * 16 + 255) / 256;
  const int dgrid = (int)(dwant < 8192 ? dwant : 8192);
  hipLaunchKernelGGL((bwd_dvec_kernel<128>), dim3(dgrid), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_fused_kernel<128>), dim3(n_cu), dim3(kMainThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// The 8-bit adder tags limit a block to 255 key blocks.
bool bwd_single_pass_supported(const BwdArgs& a, int d) {
  return d == 128 && a.n_kvblk <= kMaxAdders;
}

hipError_t launch_bwd(const BwdArgs& a, int d, hipStream_t s) {
  return d == 128 ? launch_two_pass<128, false>(a, s) : launch_two_pass<64, false>(a, s);
}

hipError_t launch_bwd_single_pass(const BwdArgs& a, int d, hipStream_t s) {
  if (!bwd_single_pass_supported(a, d)) return hipErrorInvalidValue;
  return launch_single_pass(a, s);
}

hipError_t launch_bwd_dropout(const BwdArgs& a, int d, hipStream_t s) {
  return d == 128 ? launch_two_pass<128, true>(a, s) : launch_two_pass<64, true>(a, s);
}

}  // namespace fa
