/*
 * fa.h -- C ABI of the gfx950 exact-attention library (libfa.so).
 *
 * The library computes exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T) V,     L_i = log sum_j exp(scale * q_i . k_j)  (natural log),
 * tile by tile with an online softmax, so the N_q x N_k score and probability matrices never
 * reach device memory. Sources: "Lecture 21: Optimizing Attention for Modern Hardware
 * (FlashAttention 1-4)", CMU 11-868 notes -- §0.4 (problem and notation, L = m + log l),
 * §2.2 (online softmax), §2.5 (causal masking), §2.6 (backward by recomputation, D =
 * rowsum(dO * O)), §3 (query-block parallel forward), §6.1-6.2 (split-KV decode, GQA packing);
 * "FlashAttention Tiling 策略与在线 Softmax" (ybb.press), §3 (tiled forward), §5 (backward),
 * §7 (Flash-Decoding).
 *
 * Conventions shared by every entry point
 *   Layout   Q, O, dO, dQ: [B, N_q, H_q, d] contiguous, d innermost ("BSHD").
 *            K, V, dK, dV: [B, N_k, H_kv, d] contiguous.
 *            lse (L) and the backward's D: fp32 [B, H_q, N_q] contiguous.
 *   GQA      H_q must be a multiple of H_kv; query head h reads kv head h / (H_q / H_kv).
 *   Causal   key j is visible to query i iff j <= i; requires N_q == N_k.
 *   Scale    multiplies the raw scores before the softmax; must be finite and > 0.
 *   dtype    FA_BF16: Q/K/V/O/dO/dQ/dK/dV are bfloat16, accumulation fp32, lse fp32.
 *            FA_F32 : all tensors fp32 (forward only), probabilities kept in fp32.
 *   Memory   every pointer is a device pointer owned by the caller, 16-byte aligned (the
 *            decode's int32 seqlens_k: 4-byte aligned). The library never allocates or frees
 *            memory and holds no state between calls; scratch space is a caller-provided
 *            workspace sized by the *_workspace_size queries. Calls are thread-safe.
 *   Streams  `stream` is a hipStream_t (NULL = default stream). Work is enqueued and the
 *            call returns; buffers must stay valid until the stream has passed it. Results
 *            are defined once the stream is synchronised.
 *   Errors   0 on success, a negative FA_ERR_* code otherwise. Arguments are validated on
 *            the host before any HIP call, so an invalid call has no effect. FA_ERR_HIP
 *            reports a launch failure (fa_strerror gives the HIP text); faults inside a
 *            kernel surface at the caller's next synchronisation.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_VERSION 1

enum fa_dtype { FA_F32 = 0, FA_BF16 = 1 };

enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, size < 1, H_q % H_kv != 0, bad scale, misalignment */
  FA_ERR_UNSUPPORTED = -2, /* d not in {64, 128}, dtype not supported by the call, causal with N_q != N_k */
  FA_ERR_HIP = -3,         /* a kernel launch failed */
  FA_ERR_WORKSPACE = -4,   /* workspace pointer null or smaller than the size query returned */
  FA_ERR_SCRATCH = -5      /* fa_decode_noalloc: the problem needs more than the static scratch array */
};

/*
 * Forward: O and L for Q [B,Nq,Hq,d], K/V [B,Nk,Hkv,d].
 * Per row i: m_i = max_j s_ij, l_i = sum_j exp(s_ij - m_i), O_i = sum_j exp(s_ij - m_i) v_j / l_i,
 * L_i = m_i + ln l_i (Lecture 21 notes §0.4, §2.2, §3.2). d in {64, 128}; dtype FA_BF16 or FA_F32.
 * o has Q's layout and dtype; lse is fp32 [B, Hq, Nq].
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
           int Nq, int Nk, int d, int causal, float scale, int dtype, void* stream);

/* Workspace bytes fa_fwd_persistent needs (256): its task-queue counters. They must be zero
 * before a workspace's first use (allocate it zero-filled once); every call leaves them zero
 * again, so any sequence of calls reuses one workspace without clearing. */
size_t fa_fwd_persistent_workspace_size(void);

/*
 * Persistent forward (Lecture 21 notes §4.5): the result of fa_fwd (bf16), bit for bit, from
 * one workgroup per compute unit that takes query-block tasks from a queue per XCD, in the
 * order the one-shot grid gives that XCD (without the mask a contiguous run of a head's query
 * blocks; with it longest first), and from the other XCDs' queues once its own is empty.
 * dtype FA_BF16 only (others: FA_ERR_UNSUPPORTED); d in {64, 128}. workspace: at least
 * fa_fwd_persistent_workspace_size() bytes, 16-byte aligned, zero before first use (else
 * FA_ERR_WORKSPACE if null or short). Calls that share a workspace must not overlap (one
 * stream, or synchronised).
 */
int fa_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int Nq, int Nk, int d, int causal, float scale, int dtype, void* workspace, size_t ws_bytes,
                      void* stream);

/* Workspace bytes fa_bwd needs: task-pool counters (256 bytes) and fp32 partial sums of dQ
 * (B * Hq * ceil(Nq / 64) blocks of 64 x d) at the start, then D = rowsum(dO * O) fp32
 * [B, Hq, Nq]. The first 256 + 256 * d * B * Hq * ceil(Nq / 64) bytes must be zero before a
 * workspace's first use (allocate it zero-filled once); every call leaves them zero again, so
 * calls with the same B, Hq, Nq and d reuse a workspace without clearing (the layout moves
 * with them: zero it again before a call with other values), and calls that share one must not
 * overlap. After a call that returned FA_ERR_HIP, zero it again too. D needs no initial
 * contents. */
size_t fa_bwd_workspace_size(int B, int Hq, int Nq, int d);

/*
 * Backward of f = sum(O * dO) given the forward's O and lse (Lecture 21 notes §2.6):
 * P = exp(scale*S - L) is recomputed per tile; dV = P^T dO; dP = dO V^T; dS = P * (dP - D) with
 * D = rowsum(dO * O); dQ = scale * dS K; dK = scale * dS^T Q. For GQA, dK and dV sum over the
 * query heads of a group. dtype FA_BF16 only (fp32 gives FA_ERR_UNSUPPORTED). dq has Q's layout,
 * dk and dv K's. A key-block-outer kernel forms dK and dV and a query-block-outer kernel dQ
 * (both recompute P); no atomics are involved, so results are reproducible run to run.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
           float scale, int dtype, void* workspace, size_t ws_bytes, void* stream);

/*
 * The same backward in one key-block-outer pass that forms all five products (dQ is not
 * recomputed): each 64-row block's dQ is summed in fp32 in the workspace by the key blocks in a
 * fixed order (decreasing key block, tasks taken in that order; shortest task first with the
 * causal mask), each partial sum tagged with its adder count ("Flash Attention 3/4 笔记"
 * (KaiSpace), deterministic backward; dQ accumulated over key blocks as in Lecture 21 notes
 * §2.6, exercise 6). A task only waits for tasks taken before it, so the call completes with any
 * number of its workgroups resident (other work on other streams included). Results are
 * reproducible run to run and agree with fa_bwd up to rounding. Arguments, workspace and its
 * contract as for fa_bwd. Supported: dtype FA_BF16, d = 128 and Nk <= 32640 (255 key blocks:
 * 8-bit adder tags); other shapes return FA_ERR_UNSUPPORTED before any device work. Every wait
 * for a partial sum is bounded: a wait that outlasts 0.2 s (possible only if the zeroed region
 * was not zero at the call) ends, the results of that call are then wrong, and the event is
 * counted in int32 word 15 of the workspace, which the kernel never clears (a caller that reads
 * it after the stream has passed the call sees the failure; zero the workspace before reuse).
 */
int fa_bwd_single_pass(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                       int causal, float scale, int dtype, void* workspace, size_t ws_bytes, void* stream);

/* ---- exponentials on the FMA units (Lecture 21 notes §5.2) ----
 * 2^x = 2^floor(x) * p(x - floor(x)) with p(f) = 1 + c1 f + c2 f^2 + c3 f^3, p(0) = 1, a minimax
 * fit of 2^f on [0, 1) (relative error 8.6e-5; coefficients from our own fit with Lawson's
 * algorithm, exact_io_aware_03_amd/fit_exp2.py), the power of two added to the exponent field.
 * fa_fwd_poly_exp2 is fa_fwd (bf16) with a quarter of the exponentials of every tile (one in
 * four per lane) computed this way instead of with v_exp_f32, as FA4 splits them; the result
 * agrees with fa_fwd within the bf16 rounding of P. fa_exp2_poly evaluates the same function
 * elementwise on n fp32 device values (x and y on the device; arguments below -127 give 0). */
int fa_fwd_poly_exp2(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Nq, int Nk, int d, int causal, float scale, void* stream);
int fa_exp2_poly(const float* x, float* y, long n, void* stream);

/* ---- dropout on the probabilities (Lecture 21 notes §2.8, exercise 4) ----
 * O = (P * Z / (1 - p)) V with P the normalised probabilities; lse is still the logsumexp of the
 * scores without dropout. Only the seed is kept: the keep mask Z is regenerated wherever it is
 * needed from Philox4x32-10 (Salmon et al., SC'11), one call per 4 x 4 block of (row, key)
 * positions of a (batch, query head): counter (key / 4, row / 4, b * Hq + h, offset), key (seed
 * low word, seed high word); word row % 4, byte key % 4 (little-endian) is the position's random
 * byte, kept when >= t = floor(256 p). Kept values are scaled by 256 / (256 - t), i.e. p is used
 * at 1/256 resolution. p in [0, 1) (else FA_ERR_INVALID_ARG); p < 1/256 is no dropout. bf16 only,
 * d in {64, 128}. The backward must get the forward's p, seed and offset. */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                   int Nk, int d, int causal, float scale, float p_drop, unsigned long long seed, unsigned int offset,
                   void* stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                   float scale, float p_drop, unsigned long long seed, unsigned int offset, void* workspace,
                   size_t ws_bytes, void* stream);

/* Workspace bytes fa_decode needs: arrival counters of the split sequences (ceil256(4 * B * Hq)
 * bytes at the start), then fp32 partials (o, m, l) for up to 2048 + B splits of every query
 * head. The counters must be zero before a workspace's first use (allocate it zero-filled once);
 * every call leaves them zero again, so calls with the same B and Hq reuse a workspace without
 * clearing (the layout moves with them: zero it again before a call with other values). The rest
 * of the workspace needs no initial contents. */
size_t fa_decode_workspace_size(int B, int Hq, int Nk_max, int d);

/*
 * Decode: one query per sequence against a padded KV cache (Lecture 21 notes §6.1-6.2).
 * q [B,1,Hq,d]; k_cache, v_cache [B,Nk_max,Hkv,d]; seqlens_k int32 [B] on the device: sequence b
 * attends its first seqlens_k[b] cached keys (values are clamped to [1, Nk_max]; rows past the
 * length are never read). The 64-key blocks of all sequences, in order, are cut into equal
 * contiguous ranges, one per worker of a persistent grid. A sequence that one worker covers
 * whole is finished by that worker; otherwise each worker's piece yields a partial (m, l, o) for
 * the H_q/H_kv query heads that share a kv head, and the last of the sequence's workers to
 * finish merges them by logsumexp in worker order (the result does not depend on timing). Nq
 * must be 1; dtype FA_BF16; H_q/H_kv <= 16. o [B,1,Hq,d] bf16, lse fp32 [B,Hq]. Two calls that
 * share a workspace must not overlap (one stream, or synchronised).
 */
int fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* seqlens_k, void* o,
              float* lse, int B, int Hq, int Hkv, int Nq, int Nk_max, int d, float scale, int dtype,
              void* workspace, size_t ws_bytes, void* stream);

/*
 * Decode for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same arguments and result as fa_decode minus
 * the workspace. The arrival counters and split partials live in a fixed 32 MiB device array
 * inside the library (one per GPU, zero when the library loads, held until the process ends),
 * and at most 256 workers share the block list. The counters occupy the first 512 KiB of the
 * array whatever the shape, and every call leaves them zero, so calls of any shapes follow one
 * another without clearing. A problem with B * Hq > 131072, or whose partials,
 * (256 + B) * Hq * (d + 2) * 4 bytes with the o and (m, l) parts each rounded up to 256 bytes,
 * do not fit in the remaining 31.5 MiB, returns FA_ERR_SCRATCH before any HIP call. The call
 * allocates nothing. Every call on a GPU uses that GPU's one array: calls that overlap on
 * one GPU (on two streams, or from two threads) race and must be serialised by the caller.
 */
int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* seqlens_k, void* o,
                      float* lse, int B, int Hq, int Hkv, int Nq, int Nk_max, int d, float scale, int dtype,
                      void* stream);

/* ---- FP8 forward (Lecture 21 notes §4.4 and exercise 8; "Flash Attention 3/4 笔记" §4) ----
 * Q and K in OCP E4M3 (one byte per value) with one fp32 scale per 64-row block of each
 * (batch, head), optionally rotated first by the same random orthogonal J = diag(signs) H_d /
 * sqrt(d), which leaves Q K^T unchanged and spreads outliers over all dimensions. The score
 * product runs on the FP8 MFMA; P and V stay bf16, O is bf16 and L fp32 as in fa_fwd. */

/* Number of block scales fa_quantize_fp8 writes for a [B, N, H, d] tensor: B * H * ceil(N / 64). */
size_t fa_fp8_scale_count(int B, int N, int H);

/* x: bf16 [B, N, H, d] (d in {64, 128}). signs: d fp32 values of +1 or -1 on the device, or
 * NULL for no rotation. x8: E4M3 codes [B, N, H, d]. scales: fp32 [B, H, ceil(N/64)].
 * Row r of (b, h) is multiplied by signs, transformed by the fast Walsh-Hadamard transform
 * and by 1/sqrt(d) (in fp32, in that order), then its block of 64 rows is scaled so the
 * block's largest magnitude is 448 and rounded to nearest-even E4M3: code = round(y * 448 /
 * amax), scale = amax / 448 (1 for an all-zero block); the value a code stands for is
 * decode(code) * scale. Quantise Q and K with the same signs. x and x8 16-byte aligned. */
int fa_quantize_fp8(const void* x, const float* signs, void* x8, float* scales, int B, int N, int H, int d,
                    void* stream);

/* Forward from E4M3 q8 [B,Nq,Hq,d] and k8 [B,Nk,Hkv,d] with their block scales (as written by
 * fa_quantize_fp8) and bf16 v [B,Nk,Hkv,d]: the fa_fwd result for Q = decode(q8) * q_scale and
 * K = decode(k8) * k_scale. d in {64, 128}. o bf16 [B,Nq,Hq,d], lse fp32 [B,Hq,Nq]. */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v, const float* q_scale, const float* k_scale,
               void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
               void* stream);

/* Static text for a status code (for FA_ERR_HIP: the last HIP error seen by this thread). */
const char* fa_strerror(int code);
int fa_version(void);
/* Static text naming how this library was built (target, optimisation level, the compiler's
 * scheduling strategy), so that measurements can say which build they ran. */
const char* fa_build_info(void);

/* ---- host planner helpers (pure host code; exported so the scheduling rules can be tested) ---- */

/* Fraction of CU slots busy when n_blocks equal blocks run in waves over n_cus CUs
 * (Lecture 21 notes §3.3, wave quantisation). */
double fa_wave_efficiency(int n_blocks, int n_cus);

/* Smallest split count s in [1, 128] whose wave efficiency for n_blocks*s blocks is at least
 * frac times the best over that range (Lecture 21 notes §6.1, exercise 11). frac in (0, 1],
 * else -1. */
int fa_plan_splits(int n_blocks, int n_cus, float frac);

/* Greedy list scheduling of n task lengths onto `workers`: each task goes to the least-loaded
 * worker (lowest index on ties), in arrival order or, with longest_first, longest task first
 * (Lecture 21 notes §4.5, LPT). Writes the final loads to loads_out (may be NULL) and returns
 * the makespan, or -1 on bad arguments (a negative length, or a load above INT_MAX). */
int fa_schedule_makespan(const int* w, int n, int workers, int longest_first, int* loads_out);

/* LPT: fa_schedule_makespan with the longest task first (Lecture 21 notes §4.5, exercise 10). */
int fa_lpt_makespan(const int* w, int n, int workers, int* loads_out);

/* Number of (query block, key tile) pairs a causal pass computes for N_q = N_k = n with
 * br-row query blocks and bc-key tiles, whole tiles above the diagonal skipped (§2.5). */
long fa_causal_tiles(int n, int br, int bc);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
