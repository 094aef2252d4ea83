// Single-query decode against ragged KV caches: split-KV partials + logsumexp combine.
//
// Method (Lecture 21 notes, CMU 11-868: §6.1 Flash-Decoding splits K/V along the sequence,
// each split produces a partial (m, l, o) and a small kernel merges them by the rescaling
// rule of §2.2; exercise 3: the merge is associative and commutative, so any split and any
// merge order give the same result up to rounding; §6.2 GQA packing: the query heads that
// share a K/V head are stacked as rows of one tile so K/V are read once per group).
//
// gfx950 mapping: one workgroup = (sequence b, kv head, chunk of `chunk` keys); the grid
// covers the padded maximum length and chunks past a sequence's length exit at once, so the
// ragged lengths stay on the device. The four waves take the chunk's 64-key steps in turn and
// stream them with whole-row 16-byte loads (the next step's loads in flight while this one
// computes; K staged through LDS into MFMA operand order), compute S^T = K Q^T for the
// packed query heads with v_mfma_f32_16x16x32_bf16 (query heads as the 16 MFMA columns), do
// the online softmax on the VALU, and accumulate P V on the VALU with each lane owning D/16
// head dims of one key in four. The four waves merge in LDS and write one fp32 partial per
// (query head, chunk); the combine kernel merges the partials of each (sequence, query head).
// The grid runs kv heads fastest, so the workgroups that share the cache rows of one key
// range (the kv heads are interleaved within a row) are in flight together.
// Decode is bound by HBM: every cached K/V byte is read exactly once.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kStep = 64;  // keys per wave step

__device__ __forceinline__ float xor_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float xor_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// D: head dim (64 or 128). GM: query heads per kv head the registers are sized for.
template <int D, int GM>
__global__ __launch_bounds__(kThreads, GM <= 4 ? 2 : 1) void decode_partial_kernel(DecArgs a) {
  constexpr int KS = D / 32;  // 32-dim MFMA steps
  constexpr int VE = D / 16;  // head dims per lane in the P V product
  constexpr int CH = D / 8;     // 16-byte chunks per K/V row
  constexpr int KPI = 64 / CH;  // keys per row-wise load instruction
  __shared__ __attribute__((aligned(16))) char k_lds[4][kStep * D * 2];  // per-wave K staging
  __shared__ float p_lds[4][kStep][GM];
  __shared__ float alpha_lds[4][GM];
  __shared__ float m_lds[4][GM], l_lds[4][GM];
  // the cross-wave merge reuses the K staging area once every wave has left the key loop
  static_assert(4 * GM * D * 4 <= sizeof(k_lds), "merge buffer");
  float (*o_lds)[GM][D] = reinterpret_cast<float (*)[GM][D]>(&k_lds[0][0]);

  const int hk = blockIdx.x, chunk_id = blockIdx.y, b = blockIdx.z;
  const int n = min(max(a.seqlens[b], 1), a.Nk_max);  // lengths outside [1, Nk_max] are clamped
  const int k_begin = chunk_id * a.chunk;
  if (k_begin >= n) return;  // past this sequence's length: nothing to read
  const int k_end = min(n, k_begin + a.chunk);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int G = a.G;
  const int hq0 = hk * G;

  const uint16_t* kp = (const uint16_t*)a.k + (long)b * a.Nk_max * a.k_row + hk * D;
  const uint16_t* vp = (const uint16_t*)a.v + (long)b * a.Nk_max * a.k_row + hk * D;

  // Q^T as the B operand: lane holds query head l16 (zero past G), dims [32ks + 8g4, +8).
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

  // The four waves take the chunk's 64-key steps in turn (wave w: steps w, w + 4, ...), so at
  // any moment a workgroup reads one contiguous run of cache rows.
  const int w_begin = k_begin + wave * kStep;
  const int w_end = k_end;
  constexpr int kStride = 4 * kStep;

  // K is read row-wise (CH lanes cover one key's row, KPI keys per instruction), which keeps
  // every request a whole row segment, and staged through this wave's LDS area, from where
  // the MFMA A-operand fragments (key kb*16 + l16, dims [32ks + 8g4, +8)) are read. Row
  // chunks are XOR-swizzled by key so both the row-wise stores and the fragment reads are
  // free of bank conflicts. V rows stay in registers split over 16 lanes (lane l16 owns dims
  // [VE*l16, +VE) of keys 4s + g4). Loads go through a buffer resource that ends with the
  // chunk's last key, so keys at or past w_end read as zeros without a memory access.
  u32x4 kr[CH];
  uint32_t vr[16][VE / 2];
  // per-lane part of the offsets in a VGPR, the per-instruction row step in an SGPR
  const int koff = (int)(((lane / CH) * a.k_row + (lane % CH) * 8) * 2);
  const int voff = (int)((g4 * a.k_row + l16 * VE) * 2);
  const int row_b = (int)(a.k_row * 2);
  char* kl = k_lds[wave];
  auto kswz = [](int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); };
  auto load_k = [&](int base) {
    const rsrc_t r = make_rsrc(kp + (long)base * a.k_row, ((long)(w_end - 1 - base) * a.k_row + D) * 2);
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
    const rsrc_t r = make_rsrc(vp + (long)base * a.k_row, ((long)(w_end - 1 - base) * a.k_row + D) * 2);
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

  // Software pipeline over 64-key steps: the next step's K is requested as soon as this
  // step's scores have consumed K, the next V as soon as the P V product has consumed V, so
  // each load has a whole step of arithmetic to arrive in.
  load_k(w_begin);
  load_v(w_begin);
  for (int base = w_begin; base < w_end; base += kStride) {
    stage_k();
    load_k(base + kStride);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
        if (base + kb * 16 + g4 * 4 + r >= w_end) st[kb][r] = kNegInf;
        mx = fmaxf(mx, st[kb][r]);
      }
    mx = xor_max(mx);  // all 64 keys of the step, per query head
    const float m_new = fmaxf(m, mx * a.c);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(st[kb][r], a.c, -m_use));
        rs += p;
        if (l16 < GM) p_lds[wave][kb * 16 + g4 * 4 + r][l16] = p;
      }
    l = l * alpha + rs;
    m = m_new;
    if (g4 == 0 && l16 < GM) alpha_lds[wave][l16] = alpha;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- rescale and accumulate P V ----
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      const float al = alpha_lds[wave][g];
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[g][e] *= al;
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      float pv[GM];
#pragma unroll
      for (int g = 0; g < GM; ++g) pv[g] = p_lds[wave][4 * s + g4][g];
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
    load_v(base + kStride);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four key groups of the wave, then the four waves ----
  l = xor_sum(l);
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[g][e] = xor_sum(acc[g][e]);
  __syncthreads();  // every wave is done with its K staging area, which now holds o_lds
  if (g4 == 0) {
    if (l16 < GM) {
      m_lds[wave][l16] = m;
      l_lds[wave][l16] = l;
    }
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int e = 0; e < VE; ++e) o_lds[wave][g][l16 * VE + e] = acc[g][e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int g = idx / D, dd = idx % D;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, m_lds[w][g]);
    float ll = 0.f, oo = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = fast_exp2(m_lds[w][g] - mm);  // empty waves carry m = -inf -> f = 0
      ll += f * l_lds[w][g];
      oo += f * o_lds[w][g][dd];
    }
    const long slot = ((long)b * a.Hq + hq0 + g) * a.n_chunks_max + chunk_id;
    a.part_o[slot * D + dd] = oo;
    if (dd == 0) {
      a.part_ml[slot * 2 + 0] = mm;
      a.part_ml[slot * 2 + 1] = ll;
    }
  }
}

// Merge the partials of one (sequence, query head): O = sum_c 2^(m_c - M) o_c / l,
// l = sum_c 2^(m_c - M) l_c, L = (M + log2 l) ln 2.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecArgs a) {
  const int b = blockIdx.x / a.Hq, hq = blockIdx.x % a.Hq;
  const int n = min(max(a.seqlens[b], 1), a.Nk_max);
  const int nc = (n + a.chunk - 1) / a.chunk;
  const long slot0 = ((long)b * a.Hq + hq) * a.n_chunks_max;
  float mm = kNegInf;
  for (int c = 0; c < nc; ++c) mm = fmaxf(mm, a.part_ml[(slot0 + c) * 2]);
  float ll = 0.f, oo = 0.f;
  const int dd = threadIdx.x;
  for (int c = 0; c < nc; ++c) {
    const float f = fast_exp2(a.part_ml[(slot0 + c) * 2] - mm);
    ll += f * a.part_ml[(slot0 + c) * 2 + 1];
    oo += f * a.part_o[(slot0 + c) * D + dd];
  }
  ((__bf16*)a.o)[((long)b * a.Hq + hq) * D + dd] = (__bf16)(oo / ll);
  if (dd == 0) a.lse[(long)b * a.Hq + hq] = (mm + __log2f(ll)) * kLn2;
}

template <int D>
hipError_t launch_d(const DecArgs& a, hipStream_t s) {
  const dim3 grid(a.Hkv, (a.Nk_max + a.chunk - 1) / a.chunk, a.B), block(kThreads);
  if (a.G <= 4) hipLaunchKernelGGL((decode_partial_kernel<D, 4>), grid, block, 0, s, a);
  else if (a.G <= 8) hipLaunchKernelGGL((decode_partial_kernel<D, 8>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((decode_partial_kernel<D, 16>), grid, block, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.Hq), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecArgs& a, hipStream_t s) {
  return a.d == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

}  // namespace fa
