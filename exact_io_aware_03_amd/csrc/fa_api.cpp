// C ABI of libfa: argument validation, workspace layout, planning and kernel dispatch.
// Every check runs on the host before any HIP call, so an invalid call enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <vector>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

thread_local char g_hip_msg[256] = "no HIP error recorded";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  std::snprintf(g_hip_msg, sizeof(g_hip_msg), "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return FA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int common_checks(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Dropout parameters: p must lie in [0, 1); it is used at 1/256 resolution (threshold t).
int make_dropout(float p, unsigned long long seed, unsigned int offset, fa::Dropout& dp) {
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return FA_ERR_INVALID_ARG;
  dp.t = (uint32_t)std::min(255.0, std::floor(256.0 * (double)p));
  dp.scale = (float)(256.0 / (256.0 - (double)dp.t));
  dp.k0 = (uint32_t)(seed & 0xffffffffull);
  dp.k1 = (uint32_t)(seed >> 32);
  dp.offset = offset;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_version(void) { return FA_VERSION; }

#ifndef FA_BUILD_INFO
#define FA_BUILD_INFO "unspecified build"
#endif
const char* fa_build_info(void) { return FA_BUILD_INFO; }

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or mask combination";
    case FA_ERR_HIP: return g_hip_msg;
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_SCRATCH: return "the call needs more scratch than the library's static per-GPU array holds";
    default: return "unknown status code";
  }
}

static int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int Nq, int Nk, int d, int causal, float scale, int dtype, const fa::Dropout* drop,
                      void* stream, bool poly = false, int* ctr = nullptr) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_INVALID_ARG;
  int st = common_checks(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.G = Hq / Hkv;
  a.q_row = (long)Hq * d;
  a.k_row = (long)Hkv * d;
  a.c = scale * 1.4426950408889634f;
  a.causal = causal ? 1 : 0;
  const int rows = dtype == FA_BF16 ? fa::kFwdRows : fa::kFwdF32Rows;
  a.n_qblk = (Nq + rows - 1) / rows;
  // buffer-resource offsets are 32-bit: one batch of Q/O or K/V must stay below 2 GiB
  const long esz = dtype == FA_BF16 ? 2 : 4;
  if ((long)Nq * Hq * d * esz >= (1L << 31) || (long)Nk * Hkv * d * esz >= (1L << 31)) return FA_ERR_UNSUPPORTED;
  const long tasks = (long)B * Hq * a.n_qblk;
  if (tasks > INT_MAX) return FA_ERR_INVALID_ARG;
  a.n_tasks = (int)tasks;
  hipStream_t s = (hipStream_t)stream;
  if (ctr) {
    a.ctr = ctr;
    return hip_status(fa::launch_fwd_persistent(a, d, s));
  }
  if (poly) return hip_status(fa::launch_fwd_poly(a, d, s));
  if (drop && drop->t > 0) {
    a.drop = *drop;
    return hip_status(fa::launch_fwd_dropout(a, d, s));
  }
  return hip_status(dtype == FA_BF16 ? fa::launch_fwd_bf16(a, d, s) : fa::launch_fwd_f32(a, d, s));
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
           int Nk, int d, int causal, float scale, int dtype, void* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, nullptr, stream);
}

size_t fa_fwd_persistent_workspace_size(void) { return align256(fa::kFwdPoolCounters * sizeof(int)); }

int fa_fwd_persistent(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int Nq, int Nk, int d, int causal, float scale, int dtype, void* workspace, size_t ws_bytes,
                      void* stream) {
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < fa_fwd_persistent_workspace_size() || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, nullptr, stream, false,
                    (int*)workspace);
}

int fa_fwd_poly_exp2(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Nq, int Nk, int d, int causal, float scale, void* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, FA_BF16, nullptr, stream, true);
}

int fa_exp2_poly(const float* x, float* y, long n, void* stream) {
  if (n < 0 || (n > 0 && (!x || !y))) return FA_ERR_INVALID_ARG;
  if (n == 0) return FA_OK;
  return hip_status(fa::launch_exp2_poly(x, y, n, (hipStream_t)stream));
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                   int Nk, int d, int causal, float scale, float p_drop, unsigned long long seed, unsigned int offset,
                   void* stream) {
  fa::Dropout dp{};
  const int st = make_dropout(p_drop, seed, offset, dp);
  if (st != FA_OK) return st;
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, FA_BF16, &dp, stream);
}

size_t fa_fp8_scale_count(int B, int N, int H) {
  if (B < 1 || N < 1 || H < 1) return 0;
  return (size_t)B * H * ((N + fa::kFp8Block - 1) / fa::kFp8Block);
}

int fa_quantize_fp8(const void* x, const float* signs, void* x8, float* scales, int B, int N, int H, int d,
                    void* stream) {
  if (!x || !x8 || !scales) return FA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x8) || !aligned16(scales) || (signs && !aligned16(signs))) return FA_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || H < 1) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long)B * H * ((N + fa::kFp8Block - 1) / fa::kFp8Block) > INT_MAX) return FA_ERR_INVALID_ARG;
  return hip_status(fa::launch_quantize_fp8(x, signs, x8, scales, B, N, H, d, (hipStream_t)stream));
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v, const float* q_scale, const float* k_scale, void* o,
               float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale, void* stream) {
  if (!q8 || !k8 || !v || !q_scale || !k_scale || !o || !lse) return FA_ERR_INVALID_ARG;
  for (const void* p : {q8, k8, v, (const void*)q_scale, (const void*)k_scale, (const void*)o, (const void*)lse})
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  int st = common_checks(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
  // buffer-resource offsets are 32-bit: one batch of O (bf16) or V (bf16) must stay below 2 GiB
  if ((long)Nq * Hq * d * 2 >= (1L << 31) || (long)Nk * Hkv * d * 2 >= (1L << 31)) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{};
  a.q = q8; a.k = k8; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.G = Hq / Hkv;
  a.q_row = (long)Hq * d;
  a.k_row = (long)Hkv * d;
  a.c = scale * 1.4426950408889634f;
  a.causal = causal ? 1 : 0;
  a.n_qblk = (Nq + fa::kFwdRows - 1) / fa::kFwdRows;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.q_nblk = (Nq + fa::kFp8Block - 1) / fa::kFp8Block;
  a.k_nblk = (Nk + fa::kFp8Block - 1) / fa::kFp8Block;
  const long tasks = (long)B * Hq * a.n_qblk;
  if (tasks > INT_MAX) return FA_ERR_INVALID_ARG;
  a.n_tasks = (int)tasks;
  return hip_status(fa::launch_fwd_fp8(a, d, (hipStream_t)stream));
}

// Backward workspace: the single pass's task-pool counters and its fp32 dQ partial sums (a
// 64-row x d block per query head and 64-row query block), both zero between calls, then
// D = rowsum(dO * O) [B, Hq, Nq]. Returns the total bytes; fills the parts when a is given.
static size_t bwd_zeroed_bytes(int B, int Hq, int Nq, int d) {
  const size_t blocks = (size_t)B * Hq * ((Nq + fa::kBwdRows - 1) / fa::kBwdRows);
  return align256(fa::kBwdPoolCounters * sizeof(int)) + blocks * fa::kBwdRows * d * sizeof(float);
}

static size_t bwd_layout(int B, int Hq, int Nq, int d, void* base, fa::BwdArgs* a) {
  const size_t z_bytes = bwd_zeroed_bytes(B, Hq, Nq, d);
  const size_t d_bytes = align256((size_t)B * Hq * Nq * sizeof(float));
  if (a) {
    char* p = (char*)base;
    a->ctr = (int*)p;
    a->dq_acc = (float*)(p + align256(fa::kBwdPoolCounters * sizeof(int)));
    a->dvec = (float*)(p + z_bytes);
  }
  return z_bytes + d_bytes;
}

size_t fa_bwd_workspace_size(int B, int Hq, int Nq, int d) {
  if (B < 1 || Hq < 1 || Nq < 1 || d < 1) return 0;
  return bwd_layout(B, Hq, Nq, d, nullptr, nullptr);
}

static int bwd_common(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                      float scale, int dtype, void* workspace, size_t ws_bytes, const fa::Dropout* drop,
                      bool single_pass, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, o, dout, (const void*)lse, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  int st = common_checks(B, Hq, Hkv, Nq, Nk, d, scale);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (causal && Nq != Nk) return FA_ERR_UNSUPPORTED;
  // buffer-resource offsets are 32-bit: one batch of Q/dO or K/V must stay below 2 GiB
  if ((long)Nq * Hq * d * 2 >= (1L << 31) || (long)Nk * Hkv * d * 2 >= (1L << 31)) return FA_ERR_UNSUPPORTED;
  const size_t need = fa_bwd_workspace_size(B, Hq, Nq, d);
  if (!workspace || ws_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  fa::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  bwd_layout(B, Hq, Nq, d, workspace, &a);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.G = Hq / Hkv;
  a.q_row = (long)Hq * d;
  a.k_row = (long)Hkv * d;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  a.causal = causal ? 1 : 0;
  a.n_kvblk = (Nk + fa::kBwdKeys - 1) / fa::kBwdKeys;
  a.n_qblk_dq = (Nq + fa::kBwdDqRows - 1) / fa::kBwdDqRows;
  const long tasks = (long)B * Hkv * a.n_kvblk, tasks_dq = (long)B * Hq * a.n_qblk_dq;
  if (tasks > INT_MAX || tasks_dq > INT_MAX || (long)B * Nq * Hq > INT_MAX / 4) return FA_ERR_INVALID_ARG;
  if ((long)B * Hq * ((Nq + fa::kBwdRows - 1) / fa::kBwdRows) * 8 > INT_MAX / 2) return FA_ERR_INVALID_ARG;  // tiles
  a.n_tasks = (int)tasks;
  a.n_tasks_dq = (int)tasks_dq;
  if (single_pass) {
    if (!fa::bwd_single_pass_supported(a, d)) return FA_ERR_UNSUPPORTED;
    return hip_status(fa::launch_bwd_single_pass(a, d, (hipStream_t)stream));
  }
  if (drop && drop->t > 0) {
    a.drop = *drop;
    return hip_status(fa::launch_bwd_dropout(a, d, (hipStream_t)stream));
  }
  return hip_status(fa::launch_bwd(a, d, (hipStream_t)stream));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
           int dtype, void* workspace, size_t ws_bytes, void* stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, workspace,
                    ws_bytes, nullptr, false, stream);
}

int fa_bwd_single_pass(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                       int causal, float scale, int dtype, void* workspace, size_t ws_bytes, void* stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, workspace,
                    ws_bytes, nullptr, true, stream);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                   float scale, float p_drop, unsigned long long seed, unsigned int offset, void* workspace,
                   size_t ws_bytes, void* stream) {
  fa::Dropout dp{};
  const int st = make_dropout(p_drop, seed, offset, dp);
  if (st != FA_OK) return st;
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, causal, scale, FA_BF16, workspace,
                    ws_bytes, &dp, false, stream);
}

// Decode scratch layout for `workers` split workers: the arrival counters of the split
// sequences (int, room for B * Hq, of which B * Hkv are used; zero between calls; `counters`
// ints when it is given, so that the region does not move with the shape), then the fp32
// partial outputs [(workers + B) * Hq, d] and partial (max, sum) pairs [(workers + B) * Hq, 2].
// Returns the total bytes; fills the three parts when base is given.
static size_t decode_layout(int workers, int B, int Hq, int d, void* base, fa::DecArgs* a, int counters = 0) {
  const size_t slots = (size_t)(workers + B) * Hq;
  const size_t c_bytes = align256((size_t)(counters > 0 ? counters : (long)B * Hq) * sizeof(int));
  const size_t o_bytes = align256(slots * d * sizeof(float)), ml_bytes = align256(slots * 2 * sizeof(float));
  if (base && a) {
    a->arrive = (int*)base;
    a->part_o = (float*)((char*)base + c_bytes);
    a->part_ml = (float*)((char*)base + c_bytes + o_bytes);
  }
  return c_bytes + o_bytes + ml_bytes;
}

size_t fa_decode_workspace_size(int B, int Hq, int Nk_max, int d) {
  if (B < 1 || Hq < 1 || Nk_max < 1 || d < 1) return 0;
  return decode_layout(fa::kDecMaxWorkers, B, Hq, d, nullptr, nullptr);
}

// Validation shared by the decode entry points; fills everything but the scratch pointers.
static int decode_setup(const void* q, const void* k_cache, const void* v_cache, const int* seqlens_k, void* o,
                        float* lse, int B, int Hq, int Hkv, int Nq, int Nk_max, int d, float scale, int dtype,
                        fa::DecArgs& a) {
  if (!q || !k_cache || !v_cache || !seqlens_k || !o || !lse) return FA_ERR_INVALID_ARG;
  for (const void* p : {q, k_cache, v_cache, (const void*)o, (const void*)lse})
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(seqlens_k) & 3u) != 0) return FA_ERR_INVALID_ARG;
  if (Nq != 1) return FA_ERR_INVALID_ARG;
  int st = common_checks(B, Hq, Hkv, 1, Nk_max, d, scale);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16 || Hq / Hkv > 16) return FA_ERR_UNSUPPORTED;
  if ((long)B * Nk_max * Hkv > INT_MAX / 128) return FA_ERR_INVALID_ARG;
  // the partials are addressed with 32-bit buffer offsets
  if ((long)(fa::kDecMaxWorkers + B) * Hq * d * 4 >= (1L << 31)) return FA_ERR_UNSUPPORTED;
  a = fa::DecArgs{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.seqlens = seqlens_k; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.Nk_max = Nk_max; a.d = d;
  a.k_row = (long)Hkv * d;
  a.c = scale * 1.4426950408889634f;
  return FA_OK;
}

int fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* seqlens_k, void* o, float* lse,
              int B, int Hq, int Hkv, int Nq, int Nk_max, int d, float scale, int dtype, void* workspace,
              size_t ws_bytes, void* stream) {
  fa::DecArgs a;
  const int st = decode_setup(q, k_cache, v_cache, seqlens_k, o, lse, B, Hq, Hkv, Nq, Nk_max, d, scale, dtype, a);
  if (st != FA_OK) return st;
  const size_t need = fa_decode_workspace_size(B, Hq, Nk_max, d);
  if (!workspace || ws_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  decode_layout(fa::kDecMaxWorkers, B, Hq, d, workspace, &a);
  a.max_workers = fa::kDecMaxWorkers;
  return hip_status(fa::launch_decode(a, (hipStream_t)stream));
}

int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int* seqlens_k, void* o,
                      float* lse, int B, int Hq, int Hkv, int Nq, int Nk_max, int d, float scale, int dtype,
                      void* stream) {
  fa::DecArgs a;
  const int st = decode_setup(q, k_cache, v_cache, seqlens_k, o, lse, B, Hq, Hkv, Nq, Nk_max, d, scale, dtype, a);
  if (st != FA_OK) return st;
  // The counters keep one place in the array whatever the shape: every call leaves those it
  // used zero, and no call's partials reach them.
  if ((long)B * Hq > fa::kDecNoAllocCounters ||
      decode_layout(fa::kDecNoAllocWorkers, B, Hq, d, nullptr, nullptr, fa::kDecNoAllocCounters) >
          fa::kDecScratchBytes)
    return FA_ERR_SCRATCH;
  void* base = nullptr;
  const hipError_t e = fa::decode_scratch(&base);
  if (e != hipSuccess) return hip_status(e);
  decode_layout(fa::kDecNoAllocWorkers, B, Hq, d, base, &a, fa::kDecNoAllocCounters);
  a.max_workers = fa::kDecNoAllocWorkers;
  return hip_status(fa::launch_decode(a, (hipStream_t)stream));
}

// ---- planner helpers -------------------------------------------------------------------------

static double wave_efficiency(long n_blocks, long n_cus) {
  const long waves = (n_blocks + n_cus - 1) / n_cus;
  return (double)n_blocks / (double)(waves * n_cus);
}

double fa_wave_efficiency(int n_blocks, int n_cus) {
  if (n_blocks < 1 || n_cus < 1) return 0.0;
  return wave_efficiency(n_blocks, n_cus);
}

int fa_plan_splits(int n_blocks, int n_cus, float frac_f) {
  const double frac = (double)frac_f;
  if (n_blocks < 1 || n_cus < 1 || !(frac > 0.0) || frac > 1.0) return -1;
  constexpr int kMaxSplits = 128;
  double best = 0.0;
  for (int s = 1; s <= kMaxSplits; ++s) best = std::max(best, wave_efficiency((long)n_blocks * s, n_cus));
  for (int s = 1; s <= kMaxSplits; ++s)
    if (wave_efficiency((long)n_blocks * s, n_cus) >= frac * best) return s;
  return 1;
}

int fa_schedule_makespan(const int* w, int n, int workers, int longest_first, int* loads_out) {
  if (!w || n < 0 || workers < 1) return -1;
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  if (longest_first) std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return w[x] > w[y]; });
  std::vector<long> load(workers, 0);
  for (int idx : order) {
    if (w[idx] < 0) return -1;
    const int tgt = (int)(std::min_element(load.begin(), load.end()) - load.begin());  // lowest index on ties
    load[tgt] += w[idx];
    if (load[tgt] > INT_MAX) return -1;  // a load would not fit the int results
  }
  if (loads_out)
    for (int i = 0; i < workers; ++i) loads_out[i] = (int)load[i];
  return (int)*std::max_element(load.begin(), load.end());
}

int fa_lpt_makespan(const int* w, int n, int workers, int* loads_out) {
  return fa_schedule_makespan(w, n, workers, 1, loads_out);
}

long fa_causal_tiles(int n, int br, int bc) {
  if (n < 1 || br < 1 || bc < 1) return -1;
  long tiles = 0;
  for (int i = 0; i * br < n; ++i) {
    const int last_q = std::min(n, (i + 1) * br) - 1;
    tiles += last_q / bc + 1;
  }
  return tiles;
}

}  // extern "C"
