// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA operand conventions used throughout (CDNA3/CDNA4 32x32 and 16x16 matrix cores, wave64):
//   v_mfma_f32_32x32x16_bf16: A is 32(M) x 16(K), B is 16(K) x 32(N). Lane l supplies row
//     (A) or column (B) l%32 and the 8 consecutive K slots [8*(l/32), 8*(l/32)+8). The 32x32
//     fp32 result gives lane l column l%32 and, in register i (0..15), row
//     8*(i/4) + 4*(l/32) + i%4.
//   v_mfma_f32_16x16x32_bf16: A is 16 x 32, B is 32 x 16. Lane l supplies row/column l%16
//     and K slots [8*(l/16), 8*(l/16)+8). Result: lane l holds column l%16, rows
//     4*(l/16) + i, i = 0..3.
//   v_mfma_f32_32x32x2_f32: lane l supplies row/column l%32 and the single K slot l/32.
// A and B always assign K slots to lanes identically, so any consistent relabelling of the
// contraction index between the two operands leaves the product unchanged; the kernels use
// that freedom to hand the softmax output straight from the accumulator registers to the
// next product without a trip through LDS.
#pragma once
#include "fa_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_32x32x2f(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Reductions over the two wave halves (lane l and lane l^32) with v_permlane32_swap. Each
// of the two results holds one copy of either half's value, so max/sum of the pair is the
// reduction in every lane.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// A read-only fp32 array seen through the constant address space: uniform indexing then
// becomes a scalar load (s_load), counted by lgkmcnt, so it neither waits for nor delays the
// vector-memory loads in flight (a vector load here would make the compiler drain vmcnt).
// Only for arrays that no kernel of the launch writes.
typedef const __attribute__((address_space(4))) float cfloat;
__device__ __forceinline__ cfloat* as_cfloat(const float* p) { return (cfloat*)p; }

// Ordering point for LDS data handed between lanes of one wave (or for reusing an LDS area
// through a pointer of another type): the compiler moves no memory access across it, and the
// wavefront-scope fences make this wave's earlier LDS writes visible to its later reads. The
// hardware runs one wave's LDS instructions in order, so no workgroup barrier is needed.
__device__ __forceinline__ void wave_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  asm volatile("" ::: "memory");
}

// Raw buffer resource covering `bytes` from `base` (out-of-range loads return 0 without a
// memory access, out-of-range stores are dropped). Word 3 selects 32-bit untyped access.
// The range check applies to the 32-bit per-lane offset, so callers keep offsets below 2 GiB.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffffL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

__device__ __forceinline__ void zero16(f32x16& x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = 0.f;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x on the FMA units (Lecture 21 notes §5.2): 2^x = 2^floor(x) * 2^f, f = x - floor(x) in
// [0, 1); 2^f from the cubic 1 + c1 f + c2 f^2 + c3 f^3 (p(0) = 1, minimax relative error
// 8.6e-5 on [0, 1), fitted with Lawson's algorithm by exact_io_aware_03_amd/fit_exp2.py), and
// floor(x) added to the float's exponent field. Arguments below -127 (masked scores are -inf)
// give exactly 0.
__device__ __forceinline__ float exp2_poly(float x) {
  x = fmaxf(x, -127.f);
  const float fl = floorf(x);
  const float f = x - fl;
  const float p = fmaf(fmaf(fmaf(7.706772536e-02f, f, 2.276442498e-01f), f, 6.951169372e-01f), f, 1.f);
  return __int_as_float(__float_as_int(p) + ((int)fl << 23));
}

// Hardware dispatches consecutive workgroup ids round-robin over the 8 XCDs. Give every XCD
// one contiguous range of the task list instead, so tasks that read the same K/V rows run
// under the same L2. Bijective for any n.
__device__ __forceinline__ int xcd_contiguous_task(int wg, int n) {
  constexpr int kXcd = 8;
  const int per = n / kXcd, rem = n % kXcd;
  const int x = wg % kXcd, i = wg / kXcd;
  return x * per + (x < rem ? x : rem) + i;
}

// Index of the XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ int xcc_id() {
  int x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(x));
  return x;
}

// Causal task order over n_grp groups (heads) x n_lvl levels (level 0 = longest task). Every
// XCD keeps a fixed set of groups and works through them in clusters of `cs` groups, longest
// level first inside a cluster, with cs * n_lvl about the XCD's 32 compute units: the tasks
// sharing a group's K/V rows run together under one L2 while the long ones still start first.
// Falls back to a plain longest-first order when n_grp is not a multiple of 8. Bijective on
// [0, n_grp * n_lvl).
__device__ __forceinline__ void xcd_longest_first(int wg, int n_grp, int n_lvl, int& grp, int& lvl) {
  constexpr int kXcd = 8, kCuPerXcd = 32;
  if (n_grp % kXcd == 0) {
    const int per = n_grp / kXcd, x = wg % kXcd, i = wg / kXcd;
    int cs = 1;
    while (cs * 2 * n_lvl <= kCuPerXcd && per % (cs * 2) == 0) cs *= 2;
    const int c = i / (cs * n_lvl), r = i % (cs * n_lvl);
    lvl = r / cs;
    grp = x * per + c * cs + r % cs;
  } else {
    lvl = wg / n_grp;
    grp = wg % n_grp;
  }
}

// Row relabelling used for the A operand of the score product: swapping bits 2 and 3 of the
// row index makes accumulator register i of lane half h hold contraction index
// (i & 7) + 8*h + 16*(i >> 3), i.e. each lane half owns 8 consecutive keys per 16-key step,
// exactly the K-slot layout the next MFMA expects.
__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}


// ---- dropout mask (Lecture 21 notes §2.8: regenerate the mask from the seed) ----
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC'11): ten rounds of (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
// lo(M0 c0)) with the key advanced by the Weyl increments after every round.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    // each three-way XOR is one v_bitop3_b32 (truth table 0x96 = a ^ b ^ c)
    c = u32x4{(uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], k0, 0x96), (uint32_t)p1,
              (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], k1, 0x96), (uint32_t)p0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// One Philox call covers the 4 x 4 block of (row, key) positions (4 rg .. +3, 4 kg .. +3) of
// one (batch, query head) `bh`: counter (kg, rg, bh, offset), key (k0, k1); word r holds row
// 4 rg + r, byte c (little-endian) key 4 kg + c; a position is kept when its byte is >= t, and
// kept probabilities are multiplied by 256 / (256 - t).
__device__ __forceinline__ u32x4 drop_block(const Dropout& dp, int kg, int rg, int bh) {
  return philox4x32_10(u32x4{(uint32_t)kg, (uint32_t)rg, (uint32_t)bh, dp.offset}, dp.k0, dp.k1);
}
// Value of x in lane i ^ X of this lane's quad (DPP quad_perm).
template <int X>
__device__ __forceinline__ uint32_t quad_xor(uint32_t x) {
  constexpr int ctrl = (0 ^ X) | ((1 ^ X) << 2) | ((2 ^ X) << 4) | ((3 ^ X) << 6);
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, ctrl, 0xf, 0xf, false);
}

// Whether the position whose random byte is byte i of w is kept.
__device__ __forceinline__ bool drop_kept(const Dropout& dp, uint32_t w, int i) {
  return ((w >> (8 * i)) & 255u) >= dp.t;
}

// x where the element is kept, else 0, selected in fp32: the empty asm keeps the compiler from
// moving the select past the bf16 conversion that follows (one conversion per element and a
// perm per pair instead of one conversion per pair)
__device__ __forceinline__ float keep_or_zero(bool kept, float x) {
  float r = kept ? x : 0.f;
  asm("" : "+v"(r));
  return r;
}

// 4 x 4 transpose of words across a quad (lane r = row & 3): on entry lane r holds a[k],
// k = 0..3; on exit b[c] is lane c's a[r]. Two exchanges: with lane r ^ 1 each lane keeps
// the words of rows of its own parity and trades the others, then with lane r ^ 2 it keeps
// its own row and trades the other one; a final select puts the four words in lane order.
__device__ __forceinline__ void quad_transpose(const u32x4 a, int r, uint32_t (&b)[4]) {
  const bool odd = r & 1, hi = r & 2;
  // rows (r & 1) + 2j: kj is this lane's word, rj lane r ^ 1's
  const uint32_t k0 = odd ? a[1] : a[0], k1 = odd ? a[3] : a[2];
  const uint32_t r0 = quad_xor<1>(odd ? a[0] : a[1]), r1 = quad_xor<1>(odd ? a[2] : a[3]);
  // row r: m0 from lane r, m1 from lane r ^ 1, u0 from lane r ^ 2, u1 from lane r ^ 3
  const uint32_t m0 = hi ? k1 : k0, m1 = hi ? r1 : r0;
  const uint32_t u0 = quad_xor<2>(hi ? k0 : k1), u1 = quad_xor<2>(hi ? r0 : r1);
  const uint32_t e0 = odd ? m1 : m0, e1 = odd ? m0 : m1, f0 = odd ? u1 : u0, f1 = odd ? u0 : u1;
  b[0] = hi ? f0 : e0;
  b[1] = hi ? f1 : e1;
  b[2] = hi ? e0 : f0;
  b[3] = hi ? e1 : f1;
}

// Random words of one lane's row for the 64 keys 4 kgb .. +63 of a tile laid out as the score
// accumulators hold them (lane = query row; the four lanes of a quad are rows 4a .. 4a+3 of one
// row group and see the same keys): w[C] covers keys 4 (kgb + 4 (C >> 1) + (C & 1)) .. +3, byte
// x for key + x. The eight Philox calls are the same for the whole quad, so lane r computes
// calls r and r + 4 and the quad transposes their words.
__device__ __forceinline__ void drop_row_words(const Dropout& dp, int kgb, int row, int bh, uint32_t (&w)[8]) {
  const int a = row >> 2, r = row & 3;
  const u32x4 wa = drop_block(dp, kgb + 4 * (r >> 1) + (r & 1), a, bh);      // call c = r
  const u32x4 wb = drop_block(dp, kgb + 8 + 4 * (r >> 1) + (r & 1), a, bh);  // call c = r + 4
  uint32_t ta[4], tb[4];
  quad_transpose(wa, r, ta);
  quad_transpose(wb, r, tb);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    w[c] = ta[c];
    w[c + 4] = tb[c];
  }
}

// 4 x 4 transpose of bytes across a quad: on exit byte c of lane r is byte r of lane c's x.
// Per-lane byte selectors of v_perm (bytes 0-3 from the partner's word, 4-7 from this lane's)
// for the exchange with lane r ^ 1 and then with lane r ^ 2.
__device__ __forceinline__ uint32_t quad_transpose_bytes(uint32_t x, uint32_t sel1, uint32_t sel2) {
  const uint32_t z = __builtin_amdgcn_perm(x, quad_xor<1>(x), sel1);
  return __builtin_amdgcn_perm(z, quad_xor<2>(z), sel2);
}
__device__ __forceinline__ uint32_t quad_sel1(int r) { return (r & 1) ? 0x07030501u : 0x02060004u; }
__device__ __forceinline__ uint32_t quad_sel2(int r) { return (r & 2) ? 0x07060302u : 0x01000504u; }

// Random words of one lane's key for the 16 rows 4 rgb + 16 hi + 4 g + x, the layout of the
// dK/dV kernel's accumulators (lane = key; a quad's lanes are keys 4m .. 4m+3 and see the same
// rows): byte C = 2 hi + g of w[x] is the row's byte. The four calls are the same for the
// quad; lane r computes call r and the quad transposes the bytes of each row's word.
__device__ __forceinline__ void drop_key_words(const Dropout& dp, int rgb, int key, int bh, uint32_t (&w)[4]) {
  const int r = key & 3;
  const u32x4 c = drop_block(dp, key >> 2, rgb + 4 * (r >> 1) + (r & 1), bh);  // call r
  const uint32_t s1 = quad_sel1(r), s2 = quad_sel2(r);
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = quad_transpose_bytes(c[k], s1, s2);
}

}  // namespace fa
