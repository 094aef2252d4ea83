// FP8 quantise step for the FP8 forward: optional random-sign Hadamard rotation of each row,
// one fp32 scale per 64-row block of one (batch, head), rounding to OCP E4M3.
//
// Method (Lecture 21 notes, CMU 11-868, §4.4 and exercise 8; "Flash Attention 3/4 笔记",
// §4): per-block scales instead of one per tensor; Q and K multiplied by the same random
// orthogonal J = diag(signs) H_d / sqrt(d), which cancels in Q K^T but spreads outliers over
// all dimensions; the fast Walsh-Hadamard transform costs O(d log d) per row.
//
// gfx950 mapping: one wave per (batch, head, 64-row block), one row per lane held in
// registers; the transform is log2(d) in-register butterfly stages; the block's absolute
// maximum is a wave reduction; v_cvt_pk_fp8_f32 rounds to nearest-even E4M3 (it does not
// saturate, so values are clamped to +-448 first). The arithmetic is fixed in fp32 and in
// this order (signs, butterflies h = 1, 2, ..., d/2 as (a + b, a - b), one multiply by
// 1/sqrt(d), scale = amax / 448, code = round(clamp(y * (448 / amax)))), with contraction off,
// because the codes are integers decided by floating point.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kQThreads = 256;  // four blocks of 64 rows per workgroup

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

template <int D>
__global__ __launch_bounds__(kQThreads) void quantize_fp8_kernel(const uint16_t* x, const float* signs, uint8_t* x8,
                                                                  float* scales, int B, int N, int H) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = (N + kFp8Block - 1) / kFp8Block;
  const long unit = (long)blockIdx.x * (kQThreads / 64) + wave;  // ((b * H + h) * nb + blk)
  if (unit >= (long)B * H * nb) return;
  const int blk = (int)(unit % nb);
  const long bh = unit / nb;
  const int h = (int)(bh % H), b = (int)(bh / H);
  const int n = blk * kFp8Block + lane;
  const bool valid = n < N;
  const long row = ((long)b * N + n) * H + h;

  float y[D];
  if (valid) {
    const uint16_t* src = x + row * D;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 w = *(const u32x4*)(src + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[8 * c + 2 * e] = bf16_lo(w[e]);
        y[8 * c + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) y[i] = 0.f;
  }
  if (signs) {
#pragma unroll
    for (int i = 0; i < D; ++i) y[i] *= signs[i];
#pragma unroll
    for (int hs = 1; hs < D; hs *= 2)
#pragma unroll
      for (int i = 0; i < D; ++i)
        if (!(i & hs)) {
          const float a = y[i], c = y[i + hs];
          y[i] = a + c;
          y[i + hs] = a - c;
        }
    const float r = D == 128 ? 0.08838834764831845f : 0.125f;  // fp32 nearest to 1/sqrt(d)
#pragma unroll
    for (int i = 0; i < D; ++i) y[i] *= r;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) amax = fmaxf(amax, fabsf(y[i]));
  amax = wave_max(amax);
  const float inv = amax > 0.f ? 448.f / amax : 1.f;
  if (lane == 0) scales[unit] = amax > 0.f ? amax / 448.f : 1.f;
  if (!valid) return;
  uint8_t* dst = x8 + row * D;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = fminf(fmaxf(y[16 * c + 4 * e + t] * inv, -448.f), 448.f);
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], p, true);
      w[e] = (uint32_t)p;
    }
    *(u32x4*)(dst + 16 * c) = w;
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const void* x, const float* signs, void* x8, float* scales, int B, int N, int H,
                               int d, hipStream_t s) {
  const long units = (long)B * H * ((N + kFp8Block - 1) / kFp8Block);
  const dim3 grid((unsigned)((units + kQThreads / 64 - 1) / (kQThreads / 64))), block(kQThreads);
  if (d == 128)
    hipLaunchKernelGGL((quantize_fp8_kernel<128>), grid, block, 0, s, (const uint16_t*)x, signs, (uint8_t*)x8,
                       scales, B, N, H);
  else if (d == 64)
    hipLaunchKernelGGL((quantize_fp8_kernel<64>), grid, block, 0, s, (const uint16_t*)x, signs, (uint8_t*)x8,
                       scales, B, N, H);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa
