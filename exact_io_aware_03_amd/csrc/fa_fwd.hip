// Exact attention forward for gfx950: O = softmax(scale * Q K^T) V and the row logsumexp L.
//
// Method (Lecture 21 notes, CMU 11-868: §2.2 online softmax, §2.5 whole-tile causal skip,
// §3.1 query-block-outer loop, §3.2 deferred normalisation with only L stored, §3.4 split-Q
// across warps; "FlashAttention Tiling 策略与在线 Softmax", §3 tiling): one workgroup owns 128
// query rows, each of its four waves 32 of them; K/V tiles of 64 keys stream through LDS
// while the running max m, running sum l and the output accumulator stay in registers, so
// the N x N scores never leave the chip.
//
// gfx950 mapping:
//  * scores are computed transposed, S^T = K Q^T, so every lane owns one query: the row max
//    and row sum are in-lane reductions plus one v_permlane32_swap between the wave halves,
//    and the rescale factor alpha is a per-lane scalar;
//  * the K rows fed to the score MFMA are relabelled (bits 2 and 3 of the row swapped), which
//    leaves each lane half holding 8 consecutive keys per 16-key step: the probabilities go
//    from the score accumulator straight into the B operand of O^T += V^T P^T, no LDS trip;
//  * V is transposed once while it is written to LDS, so the A operand of the output MFMA is
//    one ds_read_b128 per lane; K and V^T tiles use XOR-swizzled 16-byte chunks so the 8
//    rows read by 8 neighbouring lanes fall in distinct banks;
//  * two LDS buffers: the global loads of tile j+2 are in flight while tile j is computed,
//    one barrier per tile;
//  * scores stay in base-2 units (scale * log2 e folded into one FMA before v_exp_f32);
//  * the rescale of the output accumulator is skipped when no row maximum moved;
//  * causal: tiles wholly above a wave's rows are skipped, diagonal tiles are masked from
//    global indices, and query blocks are scheduled longest-first inside XCD-contiguous task
//    ranges.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int BR = kFwdRows;
constexpr int BC = kFwdKeys;

template <int D>
struct Tile {
  static constexpr int KCH = D / 8;                        // 16-byte chunks per K row
  static constexpr int K_BYTES = BC * D * 2;               // K tile, row-major [key][d]
  static constexpr int V_BYTES = D * BC * 2;               // V^T tile, [d][key]
  static constexpr int BUF = K_BYTES + V_BYTES;
  static constexpr int K_ROWS_PER_PASS = kThreads / KCH;
  static constexpr int K_PASSES = BC / K_ROWS_PER_PASS;    // 16-byte K loads per thread
  static constexpr int V_BLOCKS = (BC / 4) * KCH;          // 4-key x 8-d blocks per tile
  static_assert(V_BLOCKS <= kThreads, "one V block per thread at most");
};

// Swizzle of the V^T tile: row d keeps its 8 chunks (8 keys each) XOR-permuted by
// (d ^ d>>3) & 7, distinct across both the 8 consecutive rows a read touches and the 8 rows
// one transposing write touches.
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* kp, const uint16_t* vp, long k_row, int kv0,
                                          int nk, u32x4 (&kst)[Tile<D>::K_PASSES], u32x4 (&vst)[4]) {
  using T = Tile<D>;
  const int t = threadIdx.x;
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int p = 0; p < T::K_PASSES; ++p) {
    const int key = kv0 + t / T::KCH + p * T::K_ROWS_PER_PASS;
    kst[p] = key < nk ? *(const u32x4*)(kp + (long)key * k_row + (t % T::KCH) * 8) : zero;
  }
  if (t < T::V_BLOCKS) {
    const int kg = t / T::KCH, dc = t % T::KCH;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kv0 + 4 * kg + r;
      vst[r] = key < nk ? *(const u32x4*)(vp + (long)key * k_row + dc * 8) : zero;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(char* buf, const u32x4 (&kst)[Tile<D>::K_PASSES],
                                           const u32x4 (&vst)[4]) {
  using T = Tile<D>;
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < T::K_PASSES; ++p) {
    const int row = t / T::KCH + p * T::K_ROWS_PER_PASS;
    const int ch = t % T::KCH;
    *(u32x4*)(buf + row * (D * 2) + ((ch ^ swz_perm_rows(row)) << 4)) = kst[p];
  }
  if (t < T::V_BLOCKS) {
    // Transpose the 4 keys x 8 dims block in registers: one 8-byte write per dimension.
    const int kg = t / T::KCH, dc = t % T::KCH;
    char* vt = buf + T::K_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = dc * 8 + i;
      const uint32_t w0 = vst[0][i >> 1], w1 = vst[1][i >> 1], w2 = vst[2][i >> 1], w3 = vst[3][i >> 1];
      u32x2 out;
      if (i & 1) {
        out[0] = (w0 >> 16) | (w1 & 0xffff0000u);
        out[1] = (w2 >> 16) | (w3 & 0xffff0000u);
      } else {
        out[0] = (w0 & 0xffffu) | (w1 << 16);
        out[1] = (w2 & 0xffffu) | (w3 << 16);
      }
      *(u32x2*)(vt + d * (BC * 2) + (((kg >> 1) ^ vt_swz(d)) << 4) + ((kg & 1) << 3)) = out;
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::BUF];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int task = xcd_contiguous_task(blockIdx.x, a.n_tasks);
  const int bh = task / a.n_qblk;
  const int qb = CAUSAL ? a.n_qblk - 1 - task % a.n_qblk : task % a.n_qblk;  // longest first
  const int b = bh / a.Hq, hq = bh % a.Hq, hk = hq / a.G;

  const uint16_t* qp = (const uint16_t*)a.q + (long)b * a.Nq * a.q_row + hq * D;
  const uint16_t* kp = (const uint16_t*)a.k + (long)b * a.Nk * a.k_row + hk * D;
  const uint16_t* vp = (const uint16_t*)a.v + (long)b * a.Nk * a.k_row + hk * D;

  const int q0 = qb * BR + wave * 32;  // first query row of this wave
  const int qi = q0 + l32;             // the query this lane owns

  // Q as the B operand of S^T = K Q^T: lane holds column qi, dims [16ks + 8h, +8).
  bf16x8 qf[D / 16];
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[ks] = as_bf16x8(qi < a.Nq ? *(const u32x4*)(qp + (long)qi * a.q_row + ks * 16 + h * 8) : zero);
  }

  int n_tiles = (a.Nk + BC - 1) / BC;
  if (CAUSAL) {
    const int last_q = min(a.Nq, (qb + 1) * BR) - 1;
    n_tiles = min(n_tiles, last_q / BC + 1);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = kNegInf, l = 0.f;

  u32x4 kst[T::K_PASSES], vst[4];
  load_tile<D>(kp, vp, a.k_row, 0, a.Nk, kst, vst);
  store_tile<D>(smem, kst, vst);
  if (n_tiles > 1) load_tile<D>(kp, vp, a.k_row, BC, a.Nk, kst, vst);
  __syncthreads();

  const int krow0 = swap_bits23(l32);
  for (int j = 0; j < n_tiles; ++j) {
    const char* cur = smem + (j & 1) * T::BUF;
    const int kv0 = j * BC;
    if (!CAUSAL || kv0 <= q0 + 31) {
      // ---- scores S^T = K Q^T for 64 keys (two 32-key MFMA blocks) ----
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
        const int row = 32 * kb + krow0;
        const char* kr = cur + row * (D * 2);
        const int sw = swz_perm_rows(row);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 kf = *(const bf16x8*)(kr + (((2 * ks + h) ^ sw) << 4));
          s[kb] = mfma_32x32x16(kf, qf[ks], s[kb]);
        }
      }
      // register i of block kb holds key kv0 + 32kb + (i&7) + 8h + 16(i>>3)
      if (kv0 + BC > a.Nk || (CAUSAL && kv0 + BC - 1 > q0)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kv0 + 32 * kb + (i & 7) + 8 * h + 16 * (i >> 3);
            if (key >= a.Nk || (CAUSAL && key > qi)) s[kb][i] = kNegInf;
          }
      }
      // ---- online softmax (base 2) ----
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m, mx * a.c);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(s[kb][i], a.c, -m_use));
          s[kb][i] = p;
          rs += p;
        }
      l = l * alpha + rs;  // per-half partial sum; the halves are added once at the end
      m = m_new;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      }
      // ---- O^T += V^T P^T, 16 keys per step ----
#pragma unroll
      for (int ks = 0; ks < BC / 16; ++ks) {
        const f32x16& sv = s[ks >> 1];
        const int e = (ks & 1) * 8;
        u32x4 pw;
        pw[0] = pack_bf16x2(sv[e + 0], sv[e + 1]);
        pw[1] = pack_bf16x2(sv[e + 2], sv[e + 3]);
        pw[2] = pack_bf16x2(sv[e + 4], sv[e + 5]);
        pw[3] = pack_bf16x2(sv[e + 6], sv[e + 7]);
        const bf16x8 pf = as_bf16x8(pw);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int d = 32 * db + l32;
          const bf16x8 vf =
              *(const bf16x8*)(cur + T::K_BYTES + d * (BC * 2) + (((2 * ks + h) ^ vt_swz(d)) << 4));
          o[db] = mfma_32x32x16(vf, pf, o[db]);
        }
      }
    }
    if (j + 1 < n_tiles) {
      store_tile<D>(smem + ((j + 1) & 1) * T::BUF, kst, vst);
      if (j + 2 < n_tiles) load_tile<D>(kp, vp, a.k_row, (j + 2) * BC, a.Nk, kst, vst);
    }
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, L = (m + log2 l) ln 2 ----
  l = halves_sum(l);
  if (qi < a.Nq) {
    const float inv = 1.f / l;
    uint16_t* op = (uint16_t*)a.o + ((long)b * a.Nq + qi) * a.q_row + hq * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 w;
        w[0] = pack_bf16x2(o[db][4 * jj + 0] * inv, o[db][4 * jj + 1] * inv);
        w[1] = pack_bf16x2(o[db][4 * jj + 2] * inv, o[db][4 * jj + 3] * inv);
        *(u32x2*)(op + 32 * db + 8 * jj + 4 * h) = w;
      }
    if (h == 0) a.lse[((long)b * a.Hq + hq) * a.Nq + qi] = (m + __log2f(l)) * kLn2;
  }
}

// ------------------------------------------------------------------------------------------
// fp32 forward: same schedule with true-fp32 MFMA (v_mfma_f32_32x32x2_f32) and the
// probabilities kept in fp32, since rounding P to 16 bits would cost ~1e-3 of accuracy
// (Lecture 21 notes, §5.2: bf16 P gives ~3e-3 error at N=512 vs ~3e-6 in fp32).
template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a) {
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
  const int q0 = qb * BR + wave * 32;
  const int qi = q0 + l32;

  float qf[D / 2];  // B operand of S^T = K Q^T: column qi, dim 2ks + h
#pragma unroll
  for (int ks = 0; ks < D / 2; ++ks) qf[ks] = qi < a.Nq ? qp[(long)qi * a.q_row + 2 * ks + h] : 0.f;

  int n_tiles = (a.Nk + BK - 1) / BK;
  if (a.causal) n_tiles = min(n_tiles, (min(a.Nq, (qb + 1) * BR) - 1) / BK + 1);

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = kNegInf, l = 0.f;

  for (int j = 0; j < n_tiles; ++j) {
    const int kv0 = j * BK;
    __syncthreads();
    for (int e = threadIdx.x; e < BK * D; e += kThreads) {
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

hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t s) {
  const dim3 grid(a.n_tasks), block(kThreads);
  if (d == 128) hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
