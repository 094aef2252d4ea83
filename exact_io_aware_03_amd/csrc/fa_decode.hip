// Single-query decode against ragged KV caches: split-KV partials + logsumexp combine.
//
// Method (Lecture 21 notes, CMU 11-868: §6.1 Flash-Decoding splits K/V along the sequence,
// each split produces a partial (m, l, o) and a small kernel merges them by the rescaling
// rule of §2.2; exercise 3: the merge is associative and commutative, so any split and any
// merge order give the same result up to rounding; §6.2 GQA packing: the query heads that
// share a K/V head are stacked as rows of one tile so K/V are read once per group).
//
// gfx950 mapping: a persistent grid, one workgroup per compute unit. The work is the list of
// 64-key blocks of all sequences in order (sequence 0's blocks, then sequence 1's, ...); it is
// cut into equal contiguous ranges, one per worker, so every worker streams the same number of
// bytes however ragged the lengths are, and the lengths never leave the device. A worker is a
// set of waves of one workgroup, one wave per kv head (several heads per wave when there are
// more kv heads than waves; several workers per workgroup when there are fewer): since the
// cache interleaves the kv heads within each key's row, the waves of a worker read whole
// contiguous rows between them, in step with each other when the kv heads split evenly over the
// waves. Each wave walks its range one 64-key block at a time with whole-row 16-byte loads;
// K is staged through LDS into MFMA operand order, S^T = K Q^T for the packed query heads comes
// from v_mfma_f32_16x16x32_bf16 (query heads as the 16 MFMA columns), the online softmax and
// the P V product run on the VALU (each lane owns D/16 head dims of one key in four). A wave
// writes one fp32 partial (o, m, l) per (kv head, sequence it touched): a worker's ranges and
// the sequences both advance monotonically through the block list, so (worker + sequence)
// numbers the partials without collisions. The workers that hold a sequence's first and last
// blocks record themselves, and the combine kernel merges the partials of the workers in
// between for each (sequence, query head).
// Decode is bound by HBM: every cached K/V byte is read exactly once.
#include "fa_device.h"
#include "fa_internal.h"

#include <mutex>

// Scratch of fa_decode_noalloc: the split partials and the per-sequence split bounds live here
// instead of in a caller's workspace. One copy per GPU, held until the process ends; host code
// uses only the device address hipGetSymbolAddress returns for it (decode_scratch below).
static __device__ __align__(256) unsigned char scratch[fa::kDecScratchBytes];

namespace fa {
namespace {

constexpr int kUnit = 64;  // keys per block of the work list (one wave step)

__device__ __forceinline__ float xor_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xor_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Cached length of sequence b, clamped to [1, Nk_max], and its number of 64-key blocks.
__device__ __forceinline__ int seq_len(const DecArgs& a, int b) { return min(max(a.seqlens[b], 1), a.Nk_max); }
__device__ __forceinline__ int seq_blocks(int n) { return (n + kUnit - 1) / kUnit; }

// D: head dim (64 or 128). GM: query heads per kv head the registers are sized for. NW: waves
// per workgroup (8 when GM = 4; 4 for the larger groups, whose accumulators need a SIMD's
// whole register file per wave).
template <int D, int GM, int NW>
__global__ __launch_bounds__(NW * 64, 1) void decode_partial_kernel(DecArgs a) {
  constexpr int KS = D / 32;  // 32-dim MFMA steps
  constexpr int VE = D / 16;  // head dims per lane in the P V product
  constexpr int CH = D / 8;     // 16-byte chunks per K/V row
  constexpr int KPI = 64 / CH;  // keys per row-wise load instruction
  constexpr int STAGE = kUnit * D * 2;
  // Per-wave K staging. Once the scores have read K, the same bytes hold the block's
  // probabilities p[key][head] and the rescale factors until the next block is staged.
  __shared__ __attribute__((aligned(16))) char k_lds[NW][STAGE];
  static_assert((kUnit * GM + GM) * 4 <= STAGE, "p overlay");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int G = a.G;
  // Waves side by side over kv heads; when there are fewer kv heads than waves, the workgroup
  // holds S workers.
  const int Hw = min(a.Hkv, NW), S = max(1, NW / a.Hkv);
  const int hw = wave % Hw, sub = wave / Hw;
  const int vw = (int)blockIdx.x * S + sub;  // worker index

  // ---- this worker's range [u0, u1) of the block list (every wave derives it alone) ----
  // Block indices fit in int: B * Nk_max * Hkv * 128 < 2^31 is checked on the host.
  // The first 64 sequences' block counts and their scan serve both passes (one pass over the
  // lengths when B <= 64).
  const int nb0 = lane < a.B ? seq_blocks(seq_len(a, lane)) : 0;
  const int inc0 = wave_inclusive_scan(nb0, lane);
  int U = __shfl(inc0, 63);
  for (int c0 = 64; c0 < a.B; c0 += 64) U += wave_sum(c0 + lane < a.B ? seq_blocks(seq_len(a, c0 + lane)) : 0);
  U = __builtin_amdgcn_readfirstlane(U);
  if (sub >= S) return;  // spare wave (kv heads do not divide the waves evenly)
  // never more workers than blocks, so every worker's range is non-empty
  const int W = min(a.n_workers, U);
  if (vw >= W) return;
  const int u0 = (int)((long)vw * U / W), u1 = (int)((long)(vw + 1) * U / W);
  // When the kv heads split evenly over the waves, all waves of the workgroup run the same
  // jobs and blocks; a barrier per block then keeps them reading the same cache rows at the
  // same time (measured 2% faster than letting them drift apart).
  const bool lockstep = a.Hkv % NW == 0;

  // First sequence whose blocks reach past u0, and where its blocks start.
  int b = 0, pb = 0;
  {
    int run = 0;
    for (int c0 = 0; c0 < a.B; c0 += 64) {
      const int nb = c0 == 0 ? nb0 : (c0 + lane < a.B ? seq_blocks(seq_len(a, c0 + lane)) : 0);
      const int inc = c0 == 0 ? inc0 : wave_inclusive_scan(nb, lane);
      const unsigned long long hit = __ballot(c0 + lane < a.B && run + inc > u0);
      if (hit) {
        const int ln = __builtin_ctzll(hit);
        b = c0 + ln;
        pb = run + __shfl(inc - nb, ln);
        break;
      }
      run += __shfl(inc, 63);
    }
    b = __builtin_amdgcn_readfirstlane(b);
    pb = __builtin_amdgcn_readfirstlane(pb);
  }

  // K is read row-wise (CH lanes cover one key's row, KPI keys per instruction), which keeps
  // every request a whole row segment, and staged through this wave's LDS area, from where
  // the MFMA A-operand fragments (key kb*16 + l16, dims [32ks + 8g4, +8)) are read. Row
  // chunks are XOR-swizzled by key so both the row-wise stores and the fragment reads are
  // free of bank conflicts. V rows stay in registers split over 16 lanes (lane l16 owns dims
  // [VE*l16, +VE) of keys 4s + g4). Loads go through a buffer resource that ends with the
  // job's last key, so keys at or past its end read as zeros without a memory access.
  u32x4 kr[CH];
  uint32_t vr[16][VE / 2];
  const int koff = (int)(((lane / CH) * a.k_row + (lane % CH) * 8) * 2);
  const int voff = (int)((g4 * a.k_row + l16 * VE) * 2);
  const int row_b = (int)(a.k_row * 2);
  char* kl = k_lds[wave];
  float* p_lds = reinterpret_cast<float*>(kl);  // [kUnit][GM] after the scores
  float* alpha_lds = p_lds + kUnit * GM;        // [GM]
  auto kswz = [](int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); };

  // Jobs: (sequence b, kv head hk) for each sequence the range touches and each head of the
  // wave; a job's steps are the 64-key blocks [k_lo, k_hi) of b inside the range.
  while (true) {
    const int n = seq_len(a, b);
    const int lo = max(u0, pb), hi = min(u1, pb + seq_blocks(n));
    const int k_lo = (lo - pb) * kUnit, k_hi = min(n, (hi - pb) * kUnit);
    // the workers holding a sequence's first and last blocks record themselves
    if (hw == 0 && lane == 0) {
      if (lo == pb) a.seq_w[2 * b] = vw;
      if (hi == pb + seq_blocks(n)) a.seq_w[2 * b + 1] = vw;
    }
    const long slot = (long)vw + b;
    for (int hk = hw; hk < a.Hkv; hk += Hw) {
      const uint16_t* kp = (const uint16_t*)a.k + (long)b * a.Nk_max * a.k_row + hk * D;
      const uint16_t* vp = (const uint16_t*)a.v + (long)b * a.Nk_max * a.k_row + hk * D;
      auto load_k = [&](int base) {
        const rsrc_t r = make_rsrc(kp + (long)base * a.k_row, ((long)(k_hi - 1 - base) * a.k_row + D) * 2);
#pragma unroll
        for (int i = 0; i < CH; ++i) kr[i] = __builtin_amdgcn_raw_buffer_load_b128(r, koff, i * KPI * row_b, 0);
      };
      auto stage_k = [&]() {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int key = i * KPI + lane / CH;
          *(u32x4*)(kl + key * (D * 2) + (((lane % CH) ^ kswz(key)) << 4)) = kr[i];
        }
      };
      auto load_v = [&](int base) {
        const rsrc_t r = make_rsrc(vp + (long)base * a.k_row, ((long)(k_hi - 1 - base) * a.k_row + D) * 2);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          if (VE == 8) {
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 4 * s * row_b, 0);
#pragma unroll
            for (int e = 0; e < VE / 2; ++e) vr[s][e] = t[e];
          } else {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 4 * s * row_b, 0);
#pragma unroll
            for (int e = 0; e < VE / 2; ++e) vr[s][e] = t[e];
          }
        }
      };
      // Q^T as the B operand: lane holds query head l16 (zero past G), dims [32ks + 8g4, +8).
      const int hq0 = hk * G;
      bf16x8 qf[KS];
      {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const uint16_t* qp = (const uint16_t*)a.q + ((long)b * a.Hq + hq0 + l16) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(l16 < G ? *(const u32x4*)(qp + ks * 32 + g4 * 8) : zero);
      }
      float acc[GM][VE];
#pragma unroll
      for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = 0.f;
      float m = kNegInf, l = 0.f;

      // One block at a time: its K and V are requested together and the wave waits for them.
      // Requesting the next block's K and V ahead (a software pipeline) was measured slower:
      // more bytes in flight per wave read the cache rows in a less orderly way.
      for (int base = k_lo; base < k_hi; base += kUnit) {
        if (lockstep) __syncthreads();
        load_k(base);
        load_v(base);
        stage_k();
        wave_sync();
        // ---- scores: st[kb][r] is query head l16 against key base + 16kb + 4g4 + r ----
        f32x4 st[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
          const int key = kb * 16 + l16;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const u32x4 f = *(const u32x4*)(kl + key * (D * 2) + (((4 * ks + g4) ^ kswz(key)) << 4));
            st[kb] = mfma_16x16x32(as_bf16x8(f), qf[ks], st[kb]);
          }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (base + kb * 16 + g4 * 4 + r >= k_hi) st[kb][r] = kNegInf;
            mx = fmaxf(mx, st[kb][r]);
          }
        mx = xor_max(mx);  // all 64 keys of the block, per query head
        const float m_new = fmaxf(m, mx * a.c);  // finite: the block's first key is valid
        const float alpha = fast_exp2(m - m_new);
        float rs = 0.f;
        wave_sync();  // the K fragment reads are done before p overwrites the staging
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(fmaf(st[kb][r], a.c, -m_new));
            rs += p;
            if (l16 < GM) p_lds[(kb * 16 + g4 * 4 + r) * GM + l16] = p;
          }
        l = l * alpha + rs;
        m = m_new;
        if (g4 == 0 && l16 < GM) alpha_lds[l16] = alpha;
        wave_sync();
        // ---- rescale and accumulate P V ----
#pragma unroll
        for (int g = 0; g < GM; ++g) {
          const float al = alpha_lds[g];
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[g][e] *= al;
        }
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          float pv[GM];
#pragma unroll
          for (int g = 0; g < GM; ++g) pv[g] = p_lds[(4 * s + g4) * GM + g];
#pragma unroll
          for (int e = 0; e < VE / 2; ++e) {
            const float v0 = bf16_lo(vr[s][e]), v1 = bf16_hi(vr[s][e]);
#pragma unroll
            for (int g = 0; g < GM; ++g) {
              acc[g][2 * e] = fmaf(pv[g], v0, acc[g][2 * e]);
              acc[g][2 * e + 1] = fmaf(pv[g], v1, acc[g][2 * e + 1]);
            }
          }
        }
        wave_sync();  // p and alpha are read before the next block is staged over them
      }

      // ---- the job's partial: merge the four key groups of the wave, write (o, m, l) ----
      l = xor_sum(l);
#pragma unroll
      for (int g = 0; g < GM; ++g) {
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = xor_sum(acc[g][e]);
        if (g4 == 0 && g < G) {
          float* po = a.part_o + ((slot * a.Hq) + hq0 + g) * D + l16 * VE;
#pragma unroll
          for (int e = 0; e < VE; e += 4) *(f32x4*)(po + e) = f32x4{acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]};
        }
      }
      if (g4 == 0 && l16 < G) {
        float* pm = a.part_ml + ((slot * a.Hq) + hq0 + l16) * 2;
        pm[0] = m;
        pm[1] = l;
      }
    }
    pb += seq_blocks(n);
    if (++b >= a.B || pb >= u1) break;
  }
}

// Merge the partials of one (sequence, query head), written by the workers first..last that
// covered the sequence into slots (worker + sequence): O = sum_c 2^(m_c - M) o_c / l,
// l = sum_c 2^(m_c - M) l_c, L = (M + log2 l) ln 2, with M the running maximum.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecArgs a) {
  const int b = blockIdx.x / a.Hq, hq = blockIdx.x % a.Hq;
  const int w_first = a.seq_w[2 * b], w_last = a.seq_w[2 * b + 1];
  const int dd = threadIdx.x;
  float mm = kNegInf, ll = 0.f, oo = 0.f;
  // four partials' loads in flight at a time (indices past w_last re-read w_last, unused)
  for (int w0 = w_first; w0 <= w_last; w0 += 4) {
    float mc[4], lc[4], oc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long slot = ((long)min(w0 + i, w_last) + b) * a.Hq + hq;
      mc[i] = a.part_ml[slot * 2];
      lc[i] = a.part_ml[slot * 2 + 1];
      oc[i] = a.part_o[slot * D + dd];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (w0 + i > w_last) break;
      const float mn = fmaxf(mm, mc[i]);
      const float f_old = fast_exp2(mm - mn), f_new = fast_exp2(mc[i] - mn);  // mm = -inf at first: 0
      ll = ll * f_old + lc[i] * f_new;
      oo = oo * f_old + oc[i] * f_new;
      mm = mn;
    }
  }
  ((__bf16*)a.o)[((long)b * a.Hq + hq) * D + dd] = (__bf16)(oo / ll);
  if (dd == 0) a.lse[(long)b * a.Hq + hq] = (mm + __log2f(ll)) * kLn2;
}

template <int D, int GM, int NW>
hipError_t launch_dg(DecArgs a, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int S = a.Hkv < NW ? NW / a.Hkv : 1;
  const long blocks_max = (long)a.B * ((a.Nk_max + kUnit - 1) / kUnit);
  // one workgroup per compute unit, fewer when the padded batch has fewer blocks
  long wg = cus < 1 ? 1 : cus;
  const int max_workers = a.max_workers > 0 ? a.max_workers : kDecMaxWorkers;
  if (wg > max_workers / S) wg = max_workers / S;
  if (wg > (blocks_max + S - 1) / S) wg = (blocks_max + S - 1) / S;
  if (wg < 1) wg = 1;
  a.n_workers = (int)(wg * S);
  hipLaunchKernelGGL((decode_partial_kernel<D, GM, NW>), dim3((unsigned)wg), dim3(NW * 64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.Hq), dim3(D), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecArgs& a, hipStream_t s) {
  if (a.G <= 4) return launch_dg<D, 4, 8>(a, s);
  if (a.G <= 8) return launch_dg<D, 8, 4>(a, s);
  return launch_dg<D, 16, 4>(a, s);
}

}  // namespace

hipError_t launch_decode(const DecArgs& a, hipStream_t s) {
  return a.d == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy of the array
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace fa
