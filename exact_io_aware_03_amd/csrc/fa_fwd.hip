// Exact attention forward for gfx950: O = softmax(scale * Q K^T) V and the row logsumexp L.
//
// Method (Lecture 21 notes, CMU 11-868: §2.2 online softmax, §2.5 whole-tile causal skip,
// §3.1 query-block-outer loop, §3.2 deferred normalisation with only L stored, §3.4 split-Q
// across warps, §4.3 overlap of the softmax with the matrix products, §5.3 conditional
// rescaling; "FlashAttention Tiling 策略与在线 Softmax", §3 tiling): one workgroup owns 256
// query rows of one (batch, head), each of its eight waves (two per SIMD) 32 of them; K/V tiles
// of 64 keys stream through LDS while the running max m, running sum l and the output
// accumulator stay in registers, so the N x N scores never leave the chip.
//
// gfx950 mapping:
//  * scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so every lane
//    owns one query: the row max and sum are in-lane reductions plus one v_permlane32_swap,
//    and the rescale factor alpha is a per-lane scalar;
//  * the K rows fed to the score MFMA are relabelled (bits 2 and 3 of the row swapped), which
//    leaves each lane half holding 8 consecutive keys per 16-key step: the probabilities go
//    from the score accumulator straight into the B operand of O^T += V^T P^T, no LDS trip;
//  * K/V tiles land in LDS through direct-to-LDS buffer loads (no register staging, issued as
//    inline asm so the compiler does not wait for them), three tiles ahead in a four-buffer
//    ring, one barrier per tile; K is read row-wise and V through
//    ds_read_b64_tr_b16 (the V^T operand straight from the row-major tile); each tensor's
//    16-byte chunks are XOR-swizzled by row so both read patterns are free of bank conflicts;
//  * the next tile's score MFMAs are issued in the same branch-free region as this tile's
//    exponentials and P V MFMAs, so independent MFMA and VALU work of a wave overlaps, and the
//    two waves of each SIMD fill each other's gaps;
//  * scores stay in base-2 units (scale * log2 e folded into one FMA before v_exp_f32); the
//    reference max only moves when a row's max grows by more than 2^8, so the O rescale is a
//    rare, wave-uniform branch;
//  * Q/O go through buffer instructions whose resource ends at the last valid row, so rows
//    past N read as zero and stores past N are dropped, without per-lane branches;
//  * causal: tiles wholly above a wave's rows are skipped and only the last one or two are
//    masked; tasks run longest first, each XCD keeping its own heads (one L2 per head's K/V);
//    non-causal tasks take XCD-contiguous ranges for the same reason.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 8;                // waves per workgroup, two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int QH = 1;                    // 32-row query blocks per wave
constexpr int BR = kFwdRows;             // 256 query rows per workgroup
constexpr int BC = kFwdKeys;             // 64 keys per tile
constexpr int NBUF = 4;                  // LDS tile buffers: tiles j..j+3 resident or in flight
constexpr float kTau = 8.f;              // rescale threshold, base-2 units (a factor of 256)
static_assert(BR == 32 * QH * kWaves, "rows per workgroup");
constexpr int kF32Threads = 256;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Q fragments a wave keeps in registers: bf16 (8 dims per lane per 16-dim step) or E4M3
// (32 dims per lane per 64-dim step).
template <int D, bool F8>
struct QFrag {
  typedef bf16x8 type[QH][D / 16];
};
template <int D>
struct QFrag<D, true> {
  typedef i32x8 type[QH][D / 64];
};

// One K/V tile in LDS: K row-major [key][d] in bf16, or in E4M3 (one byte per value) for the
// FP8 path, then V row-major in bf16.
template <int D, bool F8 = false>
struct Tile {
  static constexpr int KE = F8 ? 1 : 2;              // bytes per K value
  static constexpr int KROW = D * KE;                // bytes per K row
  static constexpr int ROW = D * 2;                  // bytes per V row
  static constexpr int KCH = KROW / 16, VCH = ROW / 16;  // 16-byte chunks per row
  // K area: the tile, padded to one 16-byte load per wave (an E4M3 tile at d=64 is 4 KiB; the
  // upper waves' loads then fetch nothing and fill the padding with zeros)
  static constexpr int K_BYTES = (BC * KROW < kWaves * 1024) ? kWaves * 1024 : BC * KROW;
  static constexpr int K_ROWS_LDS = K_BYTES / KROW;  // rows the K loads cover (>= BC)
  static constexpr int BUF = K_BYTES + BC * ROW;     // K tile then V tile
  static constexpr int KRR = 1024 / KROW, VRR = 1024 / ROW;  // rows one wave-wide 16-byte DMA covers
  static constexpr int KDMA = K_BYTES / 1024 / kWaves;  // DMA instructions per wave per tile (K)
  static constexpr int VDMA = BC * ROW / 1024 / kWaves;  // (V)
  static constexpr int VMCNT = KDMA + VDMA;          // DMA instructions per thread per tile
  static_assert(KDMA >= 1 && VDMA >= 1, "every wave loads part of each tensor");
};

// Chunk swizzle of the V tile, read through ds_read_b64_tr_b16 (16 lanes take a 4-row x
// 32-byte block, the wave half 4 rows x 64 bytes): XOR-ing chunk bits 2-3 with the row's
// position among 4 consecutive rows (d=128) or among 4 rows at 128-byte pitch (d=64) spreads
// the 16 chunks of a wave half over 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Chunk swizzle of the K tile, read 32 rows at a time through the row relabelling: the LDS
// serves 16 lanes of a ds_read_b128 together, so the 16 rows those lanes touch must land in 16
// distinct 16-byte bank groups -- XOR with the row's low 4 bits (d=128, 16 chunks per row) or
// with bits 1-3 (d=64, two 128-byte rows per 256-byte bank line).
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// The same for an E4M3 K tile: 128-byte rows at d=128 (two per bank line: bits 1-3) and 64-byte
// rows at d=64 (four per bank line, four chunks per row: bits 2-3).
template <int D>
__device__ __forceinline__ int k8_swz(int row) {
  return D == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
}

// Per-lane global byte offsets of the direct-to-LDS loads of one tile: the instruction p of
// wave w fills 1 KiB of LDS (region kWaves*p+w), lane i landing on row RR*region + i/KCH,
// physical chunk i%KCH; it fetches the logical chunk that the swizzle puts there.
template <int D, bool F8 = false>
struct TileDma {
  int k_off[Tile<D, F8>::KDMA];
  int v_off[Tile<D, F8>::VDMA];
  __device__ void init(long k_row) {
    using T = Tile<D, F8>;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int p = 0; p < T::KDMA; ++p) {
      const int row = T::KRR * (kWaves * p + w) + lane / T::KCH;
      const int pc = lane % T::KCH;
      const int sw = F8 ? k8_swz<D>(row) : k_swz<D>(row);
      // rows of the padding: an offset past any buffer range (zeros, no memory access)
      k_off[p] = row < BC ? (int)(row * k_row * T::KE + (pc ^ sw) * 16) : 0x7ffffff0;
    }
#pragma unroll
    for (int p = 0; p < T::VDMA; ++p) {
      const int row = T::VRR * (kWaves * p + w) + lane / T::VCH;
      const int pc = lane % T::VCH;
      v_off[p] = (int)(row * k_row * 2 + (pc ^ v_swz<D>(row)) * 16);
    }
  }
};

// Raw buffer resource as four wave-uniform scalar words (base, stride 0, size, 32-bit untyped
// format) for the inline-asm loads below; loads past `bytes` return zeros without a memory access.
__device__ __forceinline__ u32x4 dma_rsrc(const void* base, long bytes) {
  const unsigned long long p = (unsigned long long)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes <= 0 ? 0u : (bytes >= 0x7fffffffL ? 0x7fffffffu : (uint32_t)bytes));
  r[3] = 0x00020000u;
  return r;
}

// One wave-wide 16-byte direct-to-LDS load: lane i's 16 bytes land at dst + 16 i. Inline asm on
// purpose: the compiler tracks the builtin form of this load and, unable to prove that its LDS
// writes miss the tile being read, waits for every outstanding prefetch (vmcnt(0)) before the
// tile's first LDS read, which exposes the latency of the loads just issued (measured 7-8%
// slower). Completion is ordered explicitly by wait_vm_barrier; the compiler's own loads are
// drained before the first of these (its vmcnt accounting does not see them).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is written by the asm itself
__device__ __forceinline__ void lds_dma16(const u32x4& r, char* dst, int voff) {
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(size_t)((__attribute__((address_space(3))) char*)dst));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Issue the direct-to-LDS loads of the tile starting at key kv0 into `buf`; keys at or past
// nk land as zero. Completion is tracked by vmcnt (Tile::VMCNT instructions per thread).
// kp / vp: byte addresses of key 0 of this (batch, kv head); k_row: values between keys.
template <int D, bool F8>
__device__ __forceinline__ void dma_tile(char* buf, const char* kp, const char* vp, long k_row, int kv0, int nk,
                                         const TileDma<D, F8>& dm) {
  using T = Tile<D, F8>;
  // one resource over the whole head (the same for every tile, so it is formed once): values up
  // to the end of the last row; the tile's start goes into the per-lane offset, which the
  // range check covers, so keys at or past nk still read as zeros. The host keeps a head's K
  // and V below 2^31 bytes, so offset + tile start fits 32 bits unsigned (the padding rows'
  // offset included, which stays out of range)
  const long valid = (long)(nk - 1) * k_row + D;
  const u32x4 rk = dma_rsrc(kp, valid * T::KE);
  const u32x4 rv = dma_rsrc(vp, valid * 2);
  const uint32_t tk = (uint32_t)((long)kv0 * k_row * T::KE), tv = (uint32_t)((long)kv0 * k_row * 2);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int p = 0; p < T::VDMA; ++p) {
    if (p < T::KDMA) lds_dma16(rk, buf + (kWaves * p + w) * 1024, (int)((uint32_t)dm.k_off[p] + tk));
    lds_dma16(rv, buf + T::K_BYTES + (kWaves * p + w) * 1024, (int)((uint32_t)dm.v_off[p] + tv));
  }
}

// Wait until at most N vector-memory loads are outstanding and this wave's LDS reads have
// returned, then the workgroup barrier. Used instead of __syncthreads so the direct-to-LDS
// loads of later tiles stay in flight; draining LDS reads first means no wave can pass the
// barrier and refill a buffer that another wave is still reading.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
}

// Scores of this wave's rows against the 64 keys of one LDS tile: s[qh][kb] = K_kb Q_qh^T.
template <int D>
__device__ __forceinline__ void scores(const char* kt, int krow0, int h, const bf16x8 (&qf)[QH][D / 16],
                                       f32x16 (&s)[QH][2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * kb + krow0;
    const char* kr = kt + row * (D * 2);
    const int sw = k_swz<D>(row);
#pragma unroll
    for (int qh = 0; qh < QH; ++qh) zero16(s[qh][kb]);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 kf = *(const bf16x8*)(kr + (((2 * ks + h) ^ sw) << 4));
#pragma unroll
      for (int qh = 0; qh < QH; ++qh) s[qh][kb] = mfma_32x32x16(kf, qf[qh][ks], s[qh][kb]);
    }
  }
}

// The same from an E4M3 K tile and E4M3 Q fragments with v_mfma_f32_32x32x64_f8f6f4 (unit
// block scales): lane l supplies 32 consecutive dims [64 ks + 32 h, +32) of its K row and of its
// query, and the accumulator layout is that of the bf16 product, so everything downstream is
// shared. The raw scores are products of the codes; the block scales multiply them later.
__device__ __forceinline__ f32x16 mfma_32x32x64_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
template <int D>
__device__ __forceinline__ void scores_f8(const char* kt, int krow0, int h, const i32x8 (&qf)[QH][D / 64],
                                          f32x16 (&s)[QH][2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * kb + krow0;
    const char* kr = kt + row * D;
    const int sw = k8_swz<D>(row);
#pragma unroll
    for (int qh = 0; qh < QH; ++qh) zero16(s[qh][kb]);
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      const int c0 = 4 * ks + 2 * h;
      const u32x4 lo = *(const u32x4*)(kr + ((c0 ^ sw) << 4));
      const u32x4 hi = *(const u32x4*)(kr + (((c0 + 1) ^ sw) << 4));
      const i32x8 kf = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qh = 0; qh < QH; ++qh) s[qh][kb] = mfma_32x32x64_f8(kf, qf[qh][ks], s[qh][kb]);
    }
  }
}

// Register i of s[qh][kb] holds key kv0 + 32kb + (i&7) + 8h + 16(i>>3) for query q0 + 32qh + l32.
template <bool CAUSAL>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[QH][2], int kv0, int nk, int q0, int l32, int h) {
#pragma unroll
  for (int qh = 0; qh < QH; ++qh)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kv0 + 32 * kb + (i & 7) + 8 * h + 16 * (i >> 3);
        if (key >= nk || (CAUSAL && key > q0 + 32 * qh + l32)) s[qh][kb][i] = kNegInf;
      }
}

__device__ __forceinline__ float max32(const f32x16& a, const f32x16& b) {
  // two chains of three-input maxima (v_max3_f32), one per accumulator
  float x = fmaxf(fmaxf(a[0], a[1]), a[2]), y = fmaxf(fmaxf(b[0], b[1]), b[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) {
    x = fmaxf(fmaxf(x, a[i]), a[i + 1]);
    y = fmaxf(fmaxf(y, b[i]), b[i + 1]);
  }
  return fmaxf(fmaxf(x, a[15]), fmaxf(y, b[15]));
}
__device__ __forceinline__ float sum32(const f32x16& a, const f32x16& b) {
  float s0 = (a[0] + a[1]) + (a[2] + a[3]), s1 = (a[4] + a[5]) + (a[6] + a[7]);
  float s2 = (a[8] + a[9]) + (a[10] + a[11]), s3 = (a[12] + a[13]) + (a[14] + a[15]);
  float s4 = (b[0] + b[1]) + (b[2] + b[3]), s5 = (b[4] + b[5]) + (b[6] + b[7]);
  float s6 = (b[8] + b[9]) + (b[10] + b[11]), s7 = (b[12] + b[13]) + (b[14] + b[15]);
  return ((s0 + s1) + (s2 + s3)) + ((s4 + s5) + (s6 + s7));
}

// A operand of O^T += V^T P^T for d-block db and 16-key step ks, read from the row-major V tile
// with two ds_read_b64_tr_b16: in each 16-lane group, source lane s points at row r0 + s/4,
// columns c0 + 4(s%4) .. +3, and result lane i receives column c0 + i of rows r0 .. r0+3. With
// r0 = 16ks + 8h + 4rd and c0 = 32db + 16((lane/16)%2), lane l ends up with column 32db + l%32
// and keys 16ks + 8h + 0..7 -- the same K-slot order the probabilities have in the B operand.
template <int D>
__device__ __forceinline__ bf16x8 v_frag(const char* vt, int ks, int db, int lane) {
  using T = Tile<D>;
  const int s = lane & 15, g = lane >> 4;
  i16x4 r[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int row = 16 * ks + 8 * (g >> 1) + 4 * rd + (s >> 2);
    const int col_b = (32 * db + 16 * (g & 1) + 4 * (s & 3)) * 2;  // byte column
    const int off = row * T::ROW + (((col_b >> 4) ^ v_swz<D>(row)) << 4) + (col_b & 15);
    r[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + off));
  }
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 c = __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// One K/V tile of the pipelined loop for this wave's rows. On entry s holds the raw scores
// of tile j; with NEXT, the scores of tile j+1 are produced into s on exit.
// c: scale * log2(e) (times this wave's Q block scale on the FP8 path); kscale: the FP8 path's
// per-tile K block scales.
template <int D, bool CAUSAL, bool NEXT, bool F8, bool DROP, bool POLY = false>
__device__ __forceinline__ void tile_step(char* smem, int j, const char* kp, const char* vp, long k_row, int nk_load,
                                          int nk, const TileDma<D, F8>& dm, int q0, int l32, int h, int lane,
                                          int krow0, float c_in, cfloat* kscale, const Dropout& dp, int bh,
                                          const typename QFrag<D, F8>::type& qf, f32x16 (&s)[QH][2],
                                          f32x16 (&sn)[QH][2], f32x16 (&o)[QH][D / 32], float (&m)[QH],
                                          float (&l)[QH], uint32_t (&keep)[QH][8]) {
  using T = Tile<D, F8>;
  const float c = F8 ? c_in * kscale[j] : c_in;
  const int kv0 = j * BC;
  const char* cur = smem + (j % NBUF) * T::BUF;
  // buffer (j+3)%4 held tile j-1, released by the barrier that ended iteration j-1
  dma_tile<D, F8>(smem + ((j + 3) % NBUF) * T::BUF, kp, vp, k_row, (j + 3) * BC, nk_load, dm);
  if (kv0 + BC > nk || (CAUSAL && kv0 + BC - 1 > q0)) mask_tile<CAUSAL>(s, kv0, nk, q0, l32, h);

  // Conditional rescaling (Lecture 21 notes §5.3): the reference m only moves when the tile's
  // max exceeds it by more than kTau (base 2), so most tiles skip the O rescale; exponents stay
  // <= kTau and the reference cancels in O = acc / l and in L = m + log2 l. The rare rescale
  // runs first, so the exponentials, the next tile's score MFMAs and the P V MFMAs below form
  // one branch-free region that the scheduler can interleave.
  float alpha[QH], m_use[QH];
  bool moved = false;
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) {
    const float mx = halves_max(max32(s[qh][0], s[qh][1])) * c;
    const bool up = mx > m[qh] + kTau;
    const float m_new = up ? mx : m[qh];
    m_use[qh] = m_new == kNegInf ? 0.f : m_new;
    alpha[qh] = up ? fast_exp2(m[qh] - m_use[qh]) : 1.f;
    moved |= up;
    m[qh] = m_new;
  }
  if (__ballot(moved)) {
#pragma unroll
    for (int qh = 0; qh < QH; ++qh)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[qh][db][i] *= alpha[qh];
  }

  // ---- phase A: scores of tile j+1 (MFMA) interleaved with the softmax of tile j (VALU) ----
  if constexpr (NEXT) {
    if constexpr (F8) scores_f8<D>(smem + ((j + 1) % NBUF) * T::BUF, krow0, h, qf, sn);
    else scores<D>(smem + ((j + 1) % NBUF) * T::BUF, krow0, h, qf, sn);
  }
#pragma unroll
  for (int qh = 0; qh < QH; ++qh)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = fmaf(s[qh][kb][i], c, -m_use[qh]);
        // POLY: a quarter of the exponentials (FA4 takes 10-25% per row) on the FMA units
        s[qh][kb][i] = (POLY && i % 4 == 0) ? exp2_poly(x) : fast_exp2(x);
      }
  // ---- phase B: O^T += V^T P^T (MFMA) interleaved with packing and the row sums (VALU) ----
  // dropout (§2.8): byte x & 3 of keep[qh][2ks + (x >> 2)] is the random byte of key
  // kv0 + 16ks + 8h + x of this lane's row. Without the mask the words are made one tile ahead:
  // the next tile's here, while the P V MFMAs run (they do not depend on them). With the mask
  // that costs spills and the words are made for this tile, just before use.
  constexpr bool AHEAD = !CAUSAL;
  uint32_t keep_next[QH][8];
  if constexpr (DROP && AHEAD && NEXT) {
#pragma unroll
    for (int qh = 0; qh < QH; ++qh) drop_row_words(dp, (kv0 + BC + 8 * h) >> 2, q0 + 32 * qh + l32, bh, keep_next[qh]);
  }
  if constexpr (DROP && !AHEAD) {
#pragma unroll
    for (int qh = 0; qh < QH; ++qh) drop_row_words(dp, (kv0 + 8 * h) >> 2, q0 + 32 * qh + l32, bh, keep[qh]);
  }
#pragma unroll
  for (int ks = 0; ks < BC / 16; ++ks) {
    bf16x8 pf[QH];
#pragma unroll
    for (int qh = 0; qh < QH; ++qh) {
      const f32x16& sv = s[qh][ks >> 1];
      const int e = (ks & 1) * 8;
      u32x4 pw;
      if constexpr (DROP) {
        // dropout on P: this lane's 8 keys kv0 + 16ks + 8h .. +7; the row sum l keeps the
        // undropped values and 1 / (1 - p) is applied to O at the end
        float pd[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) pd[x] = keep_or_zero(drop_kept(dp, keep[qh][2 * ks + (x >> 2)], x & 3), sv[e + x]);
#pragma unroll
        for (int x = 0; x < 4; ++x) pw[x] = pack_bf16x2(pd[2 * x], pd[2 * x + 1]);
      } else {
        pw[0] = pack_bf16x2(sv[e + 0], sv[e + 1]);
        pw[1] = pack_bf16x2(sv[e + 2], sv[e + 3]);
        pw[2] = pack_bf16x2(sv[e + 4], sv[e + 5]);
        pw[3] = pack_bf16x2(sv[e + 6], sv[e + 7]);
      }
      pf[qh] = as_bf16x8(pw);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16x8 vf = v_frag<D>(cur + T::K_BYTES, ks, db, lane);
#pragma unroll
      for (int qh = 0; qh < QH; ++qh) o[qh][db] = mfma_32x32x16(vf, pf[qh], o[qh][db]);
    }
  }
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) l[qh] = l[qh] * alpha[qh] + sum32(s[qh][0], s[qh][1]);
  if constexpr (DROP && AHEAD && NEXT) {
#pragma unroll
    for (int qh = 0; qh < QH; ++qh)
#pragma unroll
      for (int c = 0; c < 8; ++c) keep[qh][c] = keep_next[qh][c];
  }

  wait_vm_barrier<T::VMCNT>();  // tile j+2 landed; tile j+3 may still be in flight
}

// One task: the query block that the one-shot grid gives workgroup `wg`.
template <int D, bool CAUSAL, bool F8, bool DROP, bool POLY = false>
__device__ __forceinline__ void fwd_body(const FwdArgs& a, char* smem, int wg) {
  using T = Tile<D, F8>;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  // Non-causal: every task costs the same; each XCD takes a contiguous run of tasks so the
  // query blocks of one head share that XCD's L2. Causal: longest first (the last row band of
  // every head, then the next band, ...) with each XCD keeping its own heads.
  int bh, qb;
  if (CAUSAL) {
    int lvl;
    xcd_longest_first(wg, a.n_tasks / a.n_qblk, a.n_qblk, bh, lvl);
    qb = a.n_qblk - 1 - lvl;
  } else {
    const int task = xcd_contiguous_task(wg, a.n_tasks);
    bh = task / a.n_qblk;
    qb = task % a.n_qblk;
  }
  const int b = bh / a.Hq, hq = bh % a.Hq, hk = hq / a.G;

  const uint16_t* qp = (const uint16_t*)a.q + (long)b * a.Nq * a.q_row + hq * D;
  const char* kp = (const char*)a.k + ((long)b * a.Nk * a.k_row + hk * D) * T::KE;
  const char* vp = (const char*)a.v + ((long)b * a.Nk * a.k_row + hk * D) * 2;
  const long q_valid = ((long)(a.Nq - 1) * a.q_row + D) * 2;

  const int q0 = qb * BR + wave * 32 * QH;  // first query row of this wave

  // Q as the B operand of S^T = K Q^T: lane holds column q0 + 32qh + l32, dims [16ks + 8h, +8)
  // (bf16) or [64ks + 32h, +32) (E4M3).
  typename QFrag<D, F8>::type qf;
  float cw = a.c;             // scale * log2(e), times the Q block scale on the FP8 path
  cfloat* ksc = nullptr;  // K block scales of this (batch, kv head), FP8 path (scalar loads)
  if constexpr (F8) {
    const char* qp8 = (const char*)a.q + (long)b * a.Nq * a.q_row + hq * D;
    const rsrc_t rq = make_rsrc(qp8, (long)(a.Nq - 1) * a.q_row + D);
#pragma unroll
    for (int qh = 0; qh < QH; ++qh)
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks) {
        const int off = (int)((long)(q0 + 32 * qh + l32) * a.q_row + ks * 64 + h * 32);
        const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
        const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0));
        qf[qh][ks] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    // rows past N (last workgroup) take the last block's scale; their output is dropped
    cw *= a.q_scale[((long)b * a.Hq + hq) * a.q_nblk + min(q0 / kFp8Block, a.q_nblk - 1)];
    ksc = as_cfloat(a.k_scale + ((long)b * a.Hkv + hk) * a.k_nblk);
  } else {
    const rsrc_t rq = make_rsrc(qp, q_valid);
#pragma unroll
    for (int qh = 0; qh < QH; ++qh)
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        qf[qh][ks] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(
            rq, (int)(((long)(q0 + 32 * qh + l32) * a.q_row + ks * 16 + h * 8) * 2), 0, 0));
  }

  int n_tiles = (a.Nk + BC - 1) / BC;
  int last_w = n_tiles - 1;  // last tile this wave computes
  if (CAUSAL) {
    n_tiles = min(n_tiles, (min(a.Nq, (qb + 1) * BR) - 1) / BC + 1);
    last_w = min(n_tiles - 1, (q0 + 32 * QH - 1) / BC);
  }
  // prefetches past the workgroup's last tile resolve to an empty buffer range (zeros, no
  // memory traffic) so every iteration issues the same number of loads
  const int nk_load = min(a.Nk, n_tiles * BC);

  f32x16 o[QH][D / 32];
#pragma unroll
  for (int qh = 0; qh < QH; ++qh)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) zero16(o[qh][db]);
  float m[QH], l[QH];
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) {
    m[qh] = kNegInf;
    l[qh] = 0.f;
  }

  // tiles 0, 1, 2 in flight; wait for 0 and 1 (the last tile's loads may stay outstanding)
  TileDma<D, F8> dm;
  dm.init(a.k_row);
  __builtin_amdgcn_s_waitcnt(0);  // the Q loads complete before the untracked tile loads start
  dma_tile<D, F8>(smem, kp, vp, a.k_row, 0, nk_load, dm);
  dma_tile<D, F8>(smem + T::BUF, kp, vp, a.k_row, BC, nk_load, dm);
  dma_tile<D, F8>(smem + 2 * T::BUF, kp, vp, a.k_row, 2 * BC, nk_load, dm);
  wait_vm_barrier<T::VMCNT>();

  const int krow0 = swap_bits23(l32);
  // scores alternate between two register sets (the loop is unrolled by two tiles), so the
  // next tile's scores never need copying
  f32x16 s0[QH][2], s1[QH][2];
  if constexpr (F8) scores_f8<D>(smem, krow0, h, qf, s0);
  else scores<D>(smem, krow0, h, qf, s0);
  uint32_t keep[QH][8] = {};  // dropout random words of the current tile (tile 0's made here)
  if constexpr (DROP && !CAUSAL) {
#pragma unroll
    for (int qh = 0; qh < QH; ++qh) drop_row_words(a.drop, (8 * h) >> 2, q0 + 32 * qh + l32, bh, keep[qh]);
  }

  // Without the mask, an odd number of look-ahead steps takes its first one before the loop
  // (its scores then move to the first register set), so the tail is the final step alone: a
  // separate look-ahead step in the tail was register-allocated with spills. With the mask the
  // look-ahead step stays in the tail (the peeled form measured 5% slower there).
  int j = 0;
  if constexpr (!CAUSAL) {
    if (last_w & 1) {
      tile_step<D, CAUSAL, true, F8, DROP, POLY>(smem, j, kp, vp, a.k_row, nk_load, a.Nk, dm, q0, l32, h, lane, krow0, cw, ksc, a.drop, bh, qf, s0, s1,
                                 o, m, l, keep);
#pragma unroll
      for (int qh = 0; qh < QH; ++qh) {
        s0[qh][0] = s1[qh][0];
        s0[qh][1] = s1[qh][1];
      }
      ++j;
    }
  }
  for (; j + 1 < last_w; j += 2) {
    tile_step<D, CAUSAL, true, F8, DROP, POLY>(smem, j, kp, vp, a.k_row, nk_load, a.Nk, dm, q0, l32, h, lane, krow0, cw, ksc, a.drop, bh, qf, s0, s1,
                               o, m, l, keep);
    tile_step<D, CAUSAL, true, F8, DROP, POLY>(smem, j + 1, kp, vp, a.k_row, nk_load, a.Nk, dm, q0, l32, h, lane, krow0, cw, ksc, a.drop, bh, qf, s1,
                               s0, o, m, l, keep);
  }
  if (CAUSAL && j < last_w) {
    tile_step<D, CAUSAL, true, F8, DROP, POLY>(smem, j, kp, vp, a.k_row, nk_load, a.Nk, dm, q0, l32, h, lane, krow0, cw, ksc, a.drop, bh, qf, s0, s1,
                               o, m, l, keep);
    ++j;
    tile_step<D, CAUSAL, false, F8, DROP, POLY>(smem, j, kp, vp, a.k_row, nk_load, a.Nk, dm, q0, l32, h, lane, krow0, cw, ksc, a.drop, bh, qf, s1,
                                s0, o, m, l, keep);
  } else {
    tile_step<D, CAUSAL, false, F8, DROP, POLY>(smem, j, kp, vp, a.k_row, nk_load, a.Nk, dm, q0, l32, h, lane, krow0, cw, ksc, a.drop, bh, qf, s0,
                                s1, o, m, l, keep);
  }
  ++j;
  // tiles past this wave's diagonal: keep the workgroup's barrier count
  for (; j < n_tiles; ++j) {
    dma_tile<D, F8>(smem + ((j + 3) % NBUF) * T::BUF, kp, vp, a.k_row, (j + 3) * BC, nk_load, dm);
    wait_vm_barrier<T::VMCNT>();
  }
  __builtin_amdgcn_s_waitcnt(0);  // drain the tail prefetches before the workgroup ends

  // ---- epilogue: O = acc / l, L = (m + log2 l) ln 2; stores past N are dropped ----
  const rsrc_t ro = make_rsrc((uint16_t*)a.o + (long)b * a.Nq * a.q_row + hq * D, q_valid);
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) {
    const float lt = halves_sum(l[qh]);
    const float inv = (DROP ? a.drop.scale : 1.f) / lt;  // dropout: kept P scaled by 1 / (1 - p)
    const int qi = q0 + 32 * qh + l32;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 w;
        w[0] = pack_bf16x2(o[qh][db][4 * jj + 0] * inv, o[qh][db][4 * jj + 1] * inv);
        w[1] = pack_bf16x2(o[qh][db][4 * jj + 2] * inv, o[qh][db][4 * jj + 3] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(
            w, ro, (int)(((long)qi * a.q_row + 32 * db + 8 * jj + 4 * h) * 2), 0, 0);
      }
    if (h == 0 && qi < a.Nq) a.lse[((long)b * a.Hq + hq) * a.Nq + qi] = (m[qh] + __log2f(lt)) * kLn2;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[NBUF * Tile<D>::BUF];
  fwd_body<D, CAUSAL, false, false>(a, smem, (int)blockIdx.x);
}

// Persistent forward (Lecture 21 notes §4.5: a persistent kernel takes its tiles from a queue
// so that one task's tail overlaps the next task's start). One workgroup per compute unit takes
// tasks from its XCD's queue, in the order the one-shot grid hands that XCD its workgroups
// (without the mask a contiguous run of query blocks, so a head's K/V rows stay in one L2; with
// it longest first within clusters of heads), then from the other XCDs' queues once its own is
// empty. Queue q holds one-shot workgroups q, q + n_pools, ...; a.ctr[q] is its head and
// a.ctr[kFwdMaxPools] counts the workgroups that have left, the last of which resets every
// counter for the next call. Each task is computed exactly as by the one-shot kernel.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_persistent_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[NBUF * Tile<D>::BUF];
  __shared__ int next_wg;
  const int np = a.n_pools, home = xcc_id() % np;
  int tried = 0;  // queues found empty (thread 0): home, home + 1, ...
  for (;;) {
    // A task is taken only once the workgroup is free: taking the next one at the start of the
    // current one hides the queue's latency but lets long causal tasks wait behind busy
    // workgroups (measured 12-15% slower with the mask).
    if (threadIdx.x == 0) {
      int wg = -1;
      while (wg < 0 && tried < np) {
        const int q = (home + tried) % np;
        const int i = __hip_atomic_fetch_add(a.ctr + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (i < (a.n_tasks - q + np - 1) / np) wg = q + np * i;
        else ++tried;
      }
      next_wg = wg;
    }
    __syncthreads();  // the previous task is done with the LDS; the next one is known
    const int wg = next_wg;
    __syncthreads();  // every wave has read it before thread 0 writes the next
    if (wg < 0) break;
    fwd_body<D, CAUSAL, false, false>(a, smem, wg);
  }
  if (threadIdx.x == 0) {
    const int fin = __hip_atomic_fetch_add(a.ctr + kFwdMaxPools, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (fin == (int)gridDim.x - 1)
      for (int q = 0; q <= kFwdMaxPools; ++q) __hip_atomic_store(a.ctr + q, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// FP8 path (Lecture 21 notes §4.4; "Flash Attention 3/4 笔记" §4): Q and K arrive as E4M3 codes
// with one scale per 64-row block (after the random-sign Hadamard rotation, which cancels in
// Q K^T); the score product runs on the FP8 MFMA at twice the bf16 rate and the block scales
// fold into the per-tile softmax multiplier. P and V stay bf16.
// Dropout on P (Lecture 21 notes §2.8): the keep mask of every (row, key) is regenerated from
// (seed, offset, batch, head, row, key) with Philox, one call per 4 x 4 block of positions.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_drop_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[NBUF * Tile<D>::BUF];
  fwd_body<D, CAUSAL, false, true>(a, smem, (int)blockIdx.x);
}

// Forward with a quarter of the exponentials from exp2_poly (Lecture 21 notes §5.2). On gfx950
// the exponential is a VALU instruction rather than a separate narrow unit, so the polynomial
// costs more issue time than the v_exp_f32 it replaces; the variant is kept to measure that and
// to pin the polynomial's accuracy inside attention.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_poly_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[NBUF * Tile<D>::BUF];
  fwd_body<D, CAUSAL, false, false, true>(a, smem, (int)blockIdx.x);
}

// y = exp2_poly(x), elementwise (for the accuracy checks of the polynomial).
__global__ __launch_bounds__(256) void exp2_poly_kernel(const float* x, float* y, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    y[i] = exp2_poly(x[i]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_fp8_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[NBUF * Tile<D, true>::BUF];
  fwd_body<D, CAUSAL, true, false>(a, smem, (int)blockIdx.x);
}

// ------------------------------------------------------------------------------------------
// fp32 forward: same schedule with true-fp32 MFMA (v_mfma_f32_32x32x2_f32) and the
// probabilities kept in fp32, since rounding P to 16 bits would cost ~1e-3 of accuracy
// (Lecture 21 notes, §5.2: bf16 P gives ~3e-3 error at N=512 vs ~3e-6 in fp32).
template <int D>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BK = kFwdF32Keys;
  __shared__ float k_lds[BK][D + 1];  // padded: 32 rows read column-wise, conflict free
  __shared__ float v_lds[BK][D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int task = xcd_contiguous_task(blockIdx.x, a.n_tasks);
  const int bh = task / a.n_qblk;
  const int qb = a.causal ? a.n_qblk - 1 - task % a.n_qblk : task % a.n_qblk;
  const int b = bh / a.Hq, hq = bh % a.Hq, hk = hq / a.G;
  const float* qp = (const float*)a.q + (long)b * a.Nq * a.q_row + hq * D;
  const float* kp = (const float*)a.k + (long)b * a.Nk * a.k_row + hk * D;
  const float* vp = (const float*)a.v + (long)b * a.Nk * a.k_row + hk * D;
  const int q0 = qb * kFwdF32Rows + wave * 32;
  const int qi = q0 + l32;

  float qf[D / 2];  // B operand of S^T = K Q^T: column qi, dim 2ks + h
#pragma unroll
  for (int ks = 0; ks < D / 2; ++ks) qf[ks] = qi < a.Nq ? qp[(long)qi * a.q_row + 2 * ks + h] : 0.f;

  int n_tiles = (a.Nk + BK - 1) / BK;
  if (a.causal) n_tiles = min(n_tiles, (min(a.Nq, (qb + 1) * kFwdF32Rows) - 1) / BK + 1);

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = kNegInf, l = 0.f;

  for (int j = 0; j < n_tiles; ++j) {
    const int kv0 = j * BK;
    __syncthreads();
    for (int e = threadIdx.x; e < BK * D; e += kF32Threads) {
      const int r = e / D, c = e % D;
      const bool ok = kv0 + r < a.Nk;
      k_lds[r][c] = ok ? kp[(long)(kv0 + r) * a.k_row + c] : 0.f;
      v_lds[r][c] = ok ? vp[(long)(kv0 + r) * a.k_row + c] : 0.f;
    }
    __syncthreads();
    if (a.causal && kv0 > q0 + 31) continue;
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) s = mfma_32x32x2f(k_lds[l32][2 * ks + h], qf[ks], s);
    // register i holds key kv0 + 8(i/4) + 4h + i%4
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kv0 + 8 * (i >> 2) + 4 * h + (i & 3);
      if (key >= a.Nk || (a.causal && key > qi)) s[i] = kNegInf;
      mx = fmaxf(mx, s[i]);
    }
    mx = halves_max(mx);
    const float m_new = fmaxf(m, mx * a.c);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = exp2f(fmaf(s[i], a.c, -m_use));
      s[i] = p;
      rs += p;
    }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    // O^T += V^T P^T, one 2-key step per accumulator register: half h feeds key 8(i/4)+4h+i%4
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = 8 * (i >> 2) + 4 * h + (i & 3);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] = mfma_32x32x2f(v_lds[kr][32 * db + l32], s[i], o[db]);
    }
  }

  l = halves_sum(l);
  if (qi < a.Nq) {
    const float inv = 1.f / l;
    float* op = (float*)a.o + ((long)b * a.Nq + qi) * a.q_row + hq * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 w;
        for (int r = 0; r < 4; ++r) w[r] = o[db][4 * jj + r] * inv;
        *(f32x4*)(op + 32 * db + 8 * jj + 4 * h) = w;
      }
    if (h == 0) a.lse[((long)b * a.Hq + hq) * a.Nq + qi] = (m + log2f(l)) * kLn2;
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t s) {
  const dim3 grid(a.n_tasks), block(kThreads);
  if (d == 128) {
    if (a.causal) hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (a.causal) hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_persistent(FwdArgs a, int d, hipStream_t s) {
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n_cu < 1) n_cu = 1;
  // one queue per XCD when the compute units split into 8 of them (the task orders assume 8)
  a.n_pools = n_cu % kFwdMaxPools == 0 ? kFwdMaxPools : 1;
  const dim3 grid(min(n_cu, a.n_tasks)), block(kThreads);
  if (d == 128) {
    if (a.causal) hipLaunchKernelGGL((fwd_persistent_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_persistent_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (a.causal) hipLaunchKernelGGL((fwd_persistent_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_persistent_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_dropout(const FwdArgs& a, int d, hipStream_t s) {
  const dim3 grid(a.n_tasks), block(kThreads);
  if (d == 128) {
    if (a.causal) hipLaunchKernelGGL((fwd_drop_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_drop_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (a.causal) hipLaunchKernelGGL((fwd_drop_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_drop_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdArgs& a, int d, hipStream_t s) {
  const dim3 grid(a.n_tasks), block(kThreads);
  if (d == 128) {
    if (a.causal) hipLaunchKernelGGL((fwd_fp8_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_fp8_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (a.causal) hipLaunchKernelGGL((fwd_fp8_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_fp8_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_poly(const FwdArgs& a, int d, hipStream_t s) {
  const dim3 grid(a.n_tasks), block(kThreads);
  if (d == 128) {
    if (a.causal) hipLaunchKernelGGL((fwd_poly_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_poly_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (a.causal) hipLaunchKernelGGL((fwd_poly_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((fwd_poly_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_exp2_poly(const float* x, float* y, long n, hipStream_t s) {
  const long want = (n + 255) / 256;
  hipLaunchKernelGGL(exp2_poly_kernel, dim3((unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096)), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t s) {
  const dim3 grid(a.n_tasks), block(kF32Threads);
  if (d == 128) hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
