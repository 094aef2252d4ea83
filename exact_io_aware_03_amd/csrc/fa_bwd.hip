// Exact attention backward for gfx950, recomputing P from the saved logsumexp.
//
// Method (Lecture 21 notes, CMU 11-868, §2.6 and exercises 4-6): the forward keeps only O and
// L = m + log l per row. The backward rebuilds each tile's P = exp(scale*S - L), forms
// dV += P^T dO, dP = dO V^T, dS = P * (dP - D) with D = rowsum(dO * O) computed by a small
// pre-kernel (sum_k P_ik dP_ik = dO_i . O_i), dK += scale dS^T Q and dQ += scale dS K. The outer
// loop runs over K/V blocks so dK and dV stay on chip and only dQ is accumulated across
// workgroups with atomic adds (half the atomics of a query-outer order).
//
// gfx950 mapping: a workgroup owns 128 keys (32 per wave) of one (batch, kv head) and walks
// the 64-row query blocks that can see them (causal: only blocks at or below the diagonal,
// longest task first), for every query head of the GQA group. Scores come out of the MFMA
// with one key per lane, so P^T and dS^T feed the dV and dK products straight from the
// accumulators (query rows relabelled as in the forward); Q and dO sit in LDS both row-major
// (score operands) and transposed (dV/dK operands); dS goes through LDS once for the dQ
// product, whose result rows map to coalesced fp32 global atomics.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int BK = kBwdKeys;  // 128 keys per workgroup
constexpr int BQ = kBwdRows;  // 64 query rows per inner step

__device__ __forceinline__ int t_swz(int d) { return (d ^ (d >> 3)) & 7; }

template <int D>
struct BwdLds {
  static constexpr int KCH = D / 8;
  static constexpr int QN = BQ * D * 2;   // Q, row-major [q][d]
  static constexpr int QT = D * BQ * 2;   // Q^T, [d][q]
  static constexpr int KT = D * BK * 2;   // K^T, [d][key]
  static constexpr int DS = BQ * BK * 2;  // dS, [q][key]
  static constexpr int OFF_QN = 0;
  static constexpr int OFF_DON = OFF_QN + QN;
  static constexpr int OFF_QT = OFF_DON + QN;
  static constexpr int OFF_DOT = OFF_QT + QT;
  static constexpr int OFF_KT = OFF_DOT + QT;
  static constexpr int OFF_DS = OFF_KT + KT;
  static constexpr int OFF_L = OFF_DS + DS;
  static constexpr int OFF_D = OFF_L + BQ * 4;
  static constexpr int BYTES = OFF_D + BQ * 4;
};

// Transpose a 4-row x 8-dim block held as four 16-byte words into eight 8-byte column
// pieces, writing them to a [dim][row] LDS array with `pitch` bytes per dim row.
__device__ __forceinline__ void write_transposed(char* base, int pitch, int rg, int dc, const u32x4 (&w)[4]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = dc * 8 + i;
    const uint32_t w0 = w[0][i >> 1], w1 = w[1][i >> 1], w2 = w[2][i >> 1], w3 = w[3][i >> 1];
    u32x2 out;
    if (i & 1) {
      out[0] = (w0 >> 16) | (w1 & 0xffff0000u);
      out[1] = (w2 >> 16) | (w3 & 0xffff0000u);
    } else {
      out[0] = (w0 & 0xffffu) | (w1 << 16);
      out[1] = (w2 & 0xffffu) | (w3 << 16);
    }
    *(u32x2*)(base + d * pitch + (((rg >> 1) ^ t_swz(d)) << 4) + ((rg & 1) << 3)) = out;
  }
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
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(BwdArgs a) {
  using L = BwdLds<D>;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  char* qn = smem + L::OFF_QN;
  char* don = smem + L::OFF_DON;
  char* qt = smem + L::OFF_QT;
  char* dot_ = smem + L::OFF_DOT;
  char* kt = smem + L::OFF_KT;
  char* dsl = smem + L::OFF_DS;
  float* l2s = (float*)(smem + L::OFF_L);
  float* dls = (float*)(smem + L::OFF_D);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int task = xcd_contiguous_task(blockIdx.x, a.n_tasks);
  const int bhk = task / a.n_kvblk, j = task % a.n_kvblk;  // j ascending: longest first
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int kv0 = j * BK;
  const int kw0 = kv0 + wave * 32;  // this wave's keys
  const int key = kw0 + l32;        // this lane's key
  const uint16_t* kp = (const uint16_t*)a.k + (long)b * a.Nk * a.k_row + hk * D;
  const uint16_t* vp = (const uint16_t*)a.v + (long)b * a.Nk * a.k_row + hk * D;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // K^T, V^T as B operands of S = Q K^T and dP = dO V^T: lane holds key, dims [16ks+8h, +8)
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bool ok = key < a.Nk;
    kf[ks] = as_bf16x8(ok ? *(const u32x4*)(kp + (long)key * a.k_row + ks * 16 + h * 8) : zero);
    vf[ks] = as_bf16x8(ok ? *(const u32x4*)(vp + (long)key * a.k_row + ks * 16 + h * 8) : zero);
  }
  // K^T of the workgroup's 128 keys into LDS for the dQ product.
  for (int blk = t; blk < (BK / 4) * L::KCH; blk += kThreads) {
    const int rg = blk / L::KCH, dc = blk % L::KCH;
    u32x4 w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = kv0 + 4 * rg + r;
      w[r] = kk < a.Nk ? *(const u32x4*)(kp + (long)kk * a.k_row + dc * 8) : zero;
    }
    write_transposed(kt, BK * 2, rg, dc, w);
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  const int n_qblk = (a.Nq + BQ - 1) / BQ;
  const int qb_first = a.causal ? kv0 / BQ : 0;
  const int arow = swap_bits23(l32);

  for (int hq = hk * a.G; hq < (hk + 1) * a.G; ++hq) {
    const uint16_t* qp = (const uint16_t*)a.q + (long)b * a.Nq * a.q_row + hq * D;
    const uint16_t* gp = (const uint16_t*)a.dout + (long)b * a.Nq * a.q_row + hq * D;
    const float* lp = a.lse + ((long)b * a.Hq + hq) * a.Nq;
    const float* dp = a.dvec + ((long)b * a.Hq + hq) * a.Nq;
    for (int qb = qb_first; qb < n_qblk; ++qb) {
      const int q0 = qb * BQ;
      // ---- stage Q and dO (row-major and transposed), L (base 2) and D ----
      for (int blk = t; blk < (BQ / 4) * L::KCH; blk += kThreads) {
        const int rg = blk / L::KCH, dc = blk % L::KCH;
        u32x4 wq[4], wg[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qq = q0 + 4 * rg + r;
          const bool ok = qq < a.Nq;
          wq[r] = ok ? *(const u32x4*)(qp + (long)qq * a.q_row + dc * 8) : zero;
          wg[r] = ok ? *(const u32x4*)(gp + (long)qq * a.q_row + dc * 8) : zero;
          const int row = 4 * rg + r;
          const int off = row * (D * 2) + ((dc ^ swz_perm_rows(row)) << 4);
          *(u32x4*)(qn + off) = wq[r];
          *(u32x4*)(don + off) = wg[r];
        }
        write_transposed(qt, BQ * 2, rg, dc, wq);
        write_transposed(dot_, BQ * 2, rg, dc, wg);
      }
      if (t < BQ) {
        const int qq = q0 + t;
        l2s[t] = qq < a.Nq ? lp[qq] * kLog2e : __builtin_inff();  // rows past Nq: P = 0
        dls[t] = qq < a.Nq ? dp[qq] : 0.f;
      }
      __syncthreads();

      const bool wave_live = !a.causal || kw0 <= q0 + BQ - 1;
      if (wave_live) {
        // ---- S = Q K^T and dP = dO V^T for 64 rows x this wave's 32 keys ----
        f32x16 s[2], g[2];
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
          for (int i = 0; i < 16; ++i) s[qh][i] = g[qh][i] = 0.f;
          const int row = 32 * qh + arow;
          const int sw = swz_perm_rows(row);
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const int off = row * (D * 2) + (((2 * ks + h) ^ sw) << 4);
            s[qh] = mfma_32x32x16(*(const bf16x8*)(qn + off), kf[ks], s[qh]);
            g[qh] = mfma_32x32x16(*(const bf16x8*)(don + off), vf[ks], g[qh]);
          }
        }
        // register i of half qh holds query row 32qh + (i&7) + 8h + 16(i>>3) and key `key`
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 32 * qh + (i & 7) + 8 * h + 16 * (i >> 3);
            float p = fast_exp2(fmaf(s[qh][i], a.c, -l2s[r]));
            if (key >= a.Nk || (a.causal && key > q0 + r)) p = 0.f;
            s[qh][i] = p;                         // P
            g[qh][i] = p * (g[qh][i] - dls[r]);  // dS
          }
        }
        // ---- dV += P^T dO, dK += dS^T Q over the 64 rows (16 per step) ----
#pragma unroll
        for (int kq = 0; kq < BQ / 16; ++kq) {
          const int e = (kq & 1) * 8;
          const f32x16& ps = s[kq >> 1];
          const f32x16& gs = g[kq >> 1];
          u32x4 pw, gw;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            pw[x] = pack_bf16x2(ps[e + 2 * x], ps[e + 2 * x + 1]);
            gw[x] = pack_bf16x2(gs[e + 2 * x], gs[e + 2 * x + 1]);
          }
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const int d = 32 * db + l32;
            const int off = d * (BQ * 2) + (((2 * kq + h) ^ t_swz(d)) << 4);
            dv[db] = mfma_32x32x16(as_bf16x8(pw), *(const bf16x8*)(dot_ + off), dv[db]);
            dk[db] = mfma_32x32x16(as_bf16x8(gw), *(const bf16x8*)(qt + off), dk[db]);
          }
        }
        // ---- dS (bf16) to LDS, row-major [q][key] for the dQ product ----
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 32 * qh + (i & 7) + 8 * h + 16 * (i >> 3);
            const int kc = wave * 32 + l32;
            *(__bf16*)(dsl + r * (BK * 2) + ((((kc >> 3) ^ (r & 7))) << 4) + ((kc & 7) << 1)) =
                (__bf16)g[qh][i];
          }
      } else {
        // all 64 rows are above this wave's keys: its dS columns are zero
        const int kc = wave * 32 + l32;
        for (int r = 32 * h; r < 32 * h + 32; ++r)
          *(__bf16*)(dsl + r * (BK * 2) + ((((kc >> 3) ^ (r & 7))) << 4) + ((kc & 7) << 1)) = (__bf16)0.f;
      }
      __syncthreads();

      // ---- dQ[64 x D] += dS[64 x 128] K[128 x D]: each wave computes 32-row x 32-dim tiles ----
      {
        constexpr int NT = 2 * (D / 32);  // output tiles
        for (int tile = wave; tile < NT; tile += 4) {
          const int qt_ = tile / (D / 32), db = tile % (D / 32);
          f32x16 acc;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[i] = 0.f;
          const int r = 32 * qt_ + l32;
          const int d = 32 * db + l32;
#pragma unroll
          for (int ks = 0; ks < BK / 16; ++ks) {
            const bf16x8 af = *(const bf16x8*)(dsl + r * (BK * 2) + (((2 * ks + h) ^ (r & 7)) << 4));
            const bf16x8 bfr = *(const bf16x8*)(kt + d * (BK * 2) + (((2 * ks + h) ^ t_swz(d)) << 4));
            acc = mfma_32x32x16(af, bfr, acc);
          }
          // register i holds row 32qt + 8(i/4) + 4h + i%4, dim d
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qq = q0 + 32 * qt_ + 8 * (i >> 2) + 4 * h + (i & 3);
            if (qq < a.Nq) unsafeAtomicAdd(a.dq_acc + (((long)b * a.Nq + qq) * a.Hq + hq) * D + d, acc[i]);
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- dK = scale * acc, dV = acc (bf16); register i holds key kw0 + 8(i/4) + 4h + i%4 ----
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = kw0 + 8 * (i >> 2) + 4 * h + (i & 3);
      if (kk < a.Nk) {
        const long off = ((long)b * a.Nk + kk) * a.k_row + hk * D + 32 * db + l32;
        ((__bf16*)a.dk)[off] = (__bf16)(dk[db][i] * a.scale);
        ((__bf16*)a.dv)[off] = (__bf16)dv[db][i];
      }
    }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.Nq * a.Hq;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((rows + 3) / 4), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_main_kernel<D>), dim3(a.n_tasks), dim3(kThreads), 0, s, a);
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
