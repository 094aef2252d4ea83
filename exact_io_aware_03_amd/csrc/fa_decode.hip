// Single-query decode against ragged KV caches: split-KV partials + logsumexp merge.
//
// Method (Lecture 21 notes, CMU 11-868: §6.1 Flash-Decoding splits K/V along the sequence,
// each split produces a partial (m, l, o) and the partials are merged by the rescaling rule of
// §2.2, with nothing to merge when a sequence was not split; exercise 3: the merge is
// associative and commutative, so any split and any merge order give the same result up to
// rounding; §6.2 GQA packing: the query heads that share a K/V head are stacked as rows of one
// tile so K/V are read once per group).
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
// the P V product run on the VALU (each lane owns D/16 head dims of one key in four). A job is
// (kv head, sequence the range touches). When one worker covers the sequence whole, it writes O
// and L itself. Otherwise it writes a partial (o, m, l) into slot (worker + sequence) -- a
// worker's ranges and the sequences both advance monotonically through the block list, so no
// two jobs share a slot -- and counts its arrival on the (sequence, kv head) counter; the last
// of the sequence's workers to arrive resets the counter and merges the partials of all of
// them in worker order, so the result does not depend on which one finishes last.
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

// Cache policy of the partials' loads and stores: sc1, coherent across the XCDs' L2 caches
// (the workers that write a sequence's partials and the one that merges them may run on any).
constexpr int kCoherent = 16;
// Cache policy of the K/V cache loads: non-temporal. Every cache byte is read exactly once, and
// streaming loads marked this way reach ~7.2 TB/s where plain ones stay near 6 (a read-only
// probe over 2 GiB); the whole call went from ~212 to ~190 us.
constexpr int kStream = 2;

// Merge the partials of sequence b for the G query heads hq0 .. hq0 + G - 1, written by the
// workers w_first .. w_last into slots (worker + b): O = sum_c 2^(m_c - M) o_c / l,
// l = sum_c 2^(m_c - M) l_c, L = (M + log2 l) ln 2, with M the running maximum (Lecture 21 §6.1,
// exercise 3), in worker order. 64 / GM lanes per head, each owning D * GM / 64 dims; four
// partials' loads are in flight at a time.
template <int D, int GM>
__device__ __forceinline__ void merge_partials(const DecArgs& a, int b, int hq0, int w_first, int w_last, int lane) {
  constexpr int LPH = 64 / GM;  // lanes per head (GM is a power of two >= G)
  constexpr int DPL = D / LPH;  // dims per lane
  const int g = lane / LPH, d0 = (lane % LPH) * DPL;
  const bool live = g < a.G;
  const long hq = (long)hq0 + (live ? g : 0);
  const long slots = (long)(a.n_workers + a.B) * a.Hq;
  const rsrc_t ro = make_rsrc(a.part_o, slots * D * 4), rm = make_rsrc(a.part_ml, slots * 2 * 4);
  float mm = kNegInf, ll = 0.f, oo[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) oo[e] = 0.f;
  for (int w0 = w_first; w0 <= w_last; w0 += 4) {
    float mc[4], lc[4], oc[4][DPL];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long slot = ((long)min(w0 + i, w_last) + b) * a.Hq + hq;  // past w_last: re-read, unused
      // (the builtins return the loaded bits as integers: reinterpret, do not convert; whole
      // 16-byte vectors are reinterpreted at once, since element-wise reinterpretation of an
      // integer vector loaded this way was compiled to one element for all)
      mc[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, (int)(slot * 8), 0, kCoherent));
      lc[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, (int)(slot * 8 + 4), 0, kCoherent));
#pragma unroll
      for (int e = 0; e < DPL; e += 4) {
        const f32x4 t = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, (int)((slot * D + d0 + e) * 4), 0, kCoherent));
#pragma unroll
        for (int x = 0; x < 4; ++x) oc[i][e + x] = t[x];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (w0 + i > w_last) break;
      const float mn = fmaxf(mm, mc[i]);
      const float f_old = fast_exp2(mm - mn), f_new = fast_exp2(mc[i] - mn);  // mm = -inf at first: 0
      ll = ll * f_old + lc[i] * f_new;
#pragma unroll
      for (int e = 0; e < DPL; ++e) oo[e] = oo[e] * f_old + oc[i][e] * f_new;
      mm = mn;
    }
  }
  if (!live) return;
  __bf16* op = (__bf16*)a.o + ((long)b * a.Hq + hq) * D + d0;
#pragma unroll
  for (int e = 0; e < DPL; ++e) op[e] = (__bf16)(oo[e] / ll);
  if (lane % LPH == 0) a.lse[(long)b * a.Hq + hq] = (mm + __log2f(ll)) * kLn2;
}

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
    const long slot = (long)vw + b;
    // the workers that cover this sequence: those holding its first and last blocks and all
    // between (worker w holds blocks [w U / W, (w + 1) U / W))
    const int w_first = (int)(((long)(pb + 1) * W - 1) / U);
    const int w_last = (int)(((long)(pb + seq_blocks(n)) * W - 1) / U);
    for (int hk = hw; hk < a.Hkv; hk += Hw) {
      const uint16_t* kp = (const uint16_t*)a.k + (long)b * a.Nk_max * a.k_row + hk * D;
      const uint16_t* vp = (const uint16_t*)a.v + (long)b * a.Nk_max * a.k_row + hk * D;
      auto load_k = [&](int base) {
        const rsrc_t r = make_rsrc(kp + (long)base * a.k_row, ((long)(k_hi - 1 - base) * a.k_row + D) * 2);
#pragma unroll
        for (int i = 0; i < CH; ++i) kr[i] = __builtin_amdgcn_raw_buffer_load_b128(r, koff, i * KPI * row_b, kStream);
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
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 4 * s * row_b, kStream);
#pragma unroll
            for (int e = 0; e < VE / 2; ++e) vr[s][e] = t[e];
          } else {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 4 * s * row_b, kStream);
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

      // ---- end of the job: merge the four key groups of the wave; the only worker of the
      //      sequence writes O and L, otherwise the partial (o, m, l) goes out and the last of
      //      the sequence's workers to arrive merges them all ----
      l = xor_sum(l);
#pragma unroll
      for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = xor_sum(acc[g][e]);
      // lane l16 < G holds m and l of query head hq0 + l16, and every lane with that l16 the
      // dims [VE l16, +VE) of all G heads
      if (w_first == w_last) {
        // Lecture 21 §6.1: a sequence that was not split needs no merge
        if (g4 == 0) {
#pragma unroll
          for (int g = 0; g < GM; ++g) {
            const float lg = __shfl(l, g);
            if (g < G) {
              uint32_t w[VE / 2];
#pragma unroll
              for (int e = 0; e < VE / 2; ++e) w[e] = pack_bf16x2(acc[g][2 * e] / lg, acc[g][2 * e + 1] / lg);
              uint16_t* op = (uint16_t*)a.o + ((long)b * a.Hq + hq0 + g) * D + l16 * VE;
              if constexpr (VE == 8) *(u32x4*)op = u32x4{w[0], w[1], w[2], w[3]};
              else *(u32x2*)op = u32x2{w[0], w[1]};
            }
          }
          if (l16 < G) a.lse[(long)b * a.Hq + hq0 + l16] = (m + __log2f(l)) * kLn2;
        }
        continue;
      }
      // partials are stored with agent-scope coherence (write-through past this XCD's L2) so
      // that the merging worker, wherever it runs, reads them from the coherent level
      if (g4 == 0) {
        const long slots = (long)(a.n_workers + a.B) * a.Hq;
        const rsrc_t ro = make_rsrc(a.part_o, slots * D * 4), rm = make_rsrc(a.part_ml, slots * 2 * 4);
#pragma unroll
        for (int g = 0; g < GM; ++g) {
          if (g < G) {
            const int off = (int)((((slot * a.Hq) + hq0 + g) * D + l16 * VE) * 4);
#pragma unroll
            for (int e = 0; e < VE; e += 4)
              __builtin_amdgcn_raw_buffer_store_b128(f32x4{acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]}, ro,
                                                     off + e * 4, 0, kCoherent);
          }
        }
        if (l16 < G)
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(m), __float_as_uint(l)}, rm,
                                                (int)(((slot * a.Hq) + hq0 + l16) * 8), 0, kCoherent);
      }
      // The stores are complete at the coherent level before the arrival is counted, and the
      // last arriver reads the partials with agent-coherent loads after its count came back;
      // that is the release/acquire pair, without the whole-cache write-back and invalidation
      // an agent-scope fence would cost (measured: the call took 1.55x as long with them).
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      int* cnt = a.arrive + (long)b * a.Hkv + hk;
      int before = 0;
      if (lane == 0) before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      before = __builtin_amdgcn_readfirstlane(__shfl(before, 0));
      if (before != w_last - w_first) continue;
      // the last to arrive: reset the counter for the next call and merge the partials of the
      // workers w_first .. w_last in that order (the result does not depend on who is last)
      if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      merge_partials<D, GM>(a, b, hq0, w_first, w_last, lane);
    }    pb += seq_blocks(n);
    if (++b >= a.B || pb >= u1) break;
  }
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
