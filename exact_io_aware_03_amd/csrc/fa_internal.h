// Host-side launch interface between the C-ABI layer (fa_api.cpp) and the kernel files.
// Everything here assumes arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Dropout on the probabilities (mask regenerated from the seed; see fa_device.h).
struct Dropout {
  uint32_t k0, k1;  // Philox key: the seed's low and high words
  uint32_t offset;  // fourth counter word (a fresh mask per call)
  uint32_t t;       // byte threshold: a position is kept when its random byte is >= t
  float scale;      // 256 / (256 - t)
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, G;
  long q_row;  // elements between consecutive positions of Q/O (Hq * d)
  long k_row;  // elements between consecutive positions of K/V (Hkv * d)
  float c;     // softmax scale * log2(e): scores are kept in base-2 units
  int causal;
  int n_qblk;   // query blocks per (batch, head)
  int n_tasks;  // B * Hq * n_qblk
  // FP8 (E4M3) Q and K only: one fp32 scale per 64-row block, [B, Hq, q_nblk] / [B, Hkv, k_nblk]
  const float* q_scale;
  const float* k_scale;
  int q_nblk, k_nblk;
  Dropout drop;  // dropout on P (bf16 path): threshold t > 0 selects the dropout instance
  // persistent forward only: task queue heads [kFwdMaxPools] and the leaver count after them,
  // zero between calls; n_pools queues (one per XCD, or one)
  int* ctr;
  int n_pools;
};

struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* seqlens;
  void* o;
  float* lse;
  float* part_o;   // [max_workers + B, Hq, d] unnormalised partial outputs
  float* part_ml;  // [max_workers + B, Hq, 2] partial (max, sum) in base-2 units
  int* arrive;     // [B, Hkv] arrival counters of the split sequences; zero between calls
  int B, Hq, Hkv, G, Nk_max, d;
  int n_workers;   // set by the launcher: workers sharing the block list
  int max_workers; // cap on n_workers (the partial slots are sized for max_workers + B per head)
  long k_row;
  float c;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;    // D = rowsum(dO * O), [B, Hq, Nq]
  // single pass only: fp32 dQ partial sums with adder tags (one 4 KiB tile per query head,
  // 64-row block and wave; zero between calls) and the task-pool counters (zero between calls)
  float* dq_acc;
  int* ctr;
  int n_pools;
  int B, Hq, Hkv, Nq, Nk, G;
  long q_row, k_row;
  float scale;
  float c;
  int causal;
  int n_kvblk;
  int n_tasks;     // dK/dV kernel: B * Hkv * n_kvblk
  int n_qblk_dq;   // dQ kernel: query blocks per (batch, head)
  int n_tasks_dq;  // B * Hq * n_qblk_dq
  Dropout drop;    // the forward's dropout, regenerated (t > 0 selects the dropout instance)
};

// Planner constants shared by the host code and the kernels.
constexpr int kFwdRows = 256;     // query rows per bf16 / fp8 forward workgroup (8 waves x 32)
constexpr int kFwdF32Rows = 128;  // query rows per fp32 forward workgroup (4 waves x 32)
constexpr int kFwdKeys = 64;      // keys per forward K/V tile
constexpr int kFwdF32Keys = 32;   // keys per tile in the fp32 forward
constexpr int kDecMaxWorkers = 2048;  // decode workers (partials per sequence boundary)
constexpr int kDecNoAllocWorkers = 256;  // worker cap of the decode that allocates nothing
constexpr size_t kDecScratchBytes = size_t(32) << 20;  // its static per-GPU scratch array
// Arrival counters at the start of that array: a region of fixed size, so that the counters of
// every problem shape lie where no call writes partials.
constexpr int kDecNoAllocCounters = 131072;
constexpr int kBwdKeys = 128;     // keys per dK/dV workgroup (4 key slices x 32)
constexpr int kBwdRows = 64;      // query rows per dK/dV inner step
constexpr int kBwdDqRows = 256;   // query rows per dQ workgroup (8 waves x 32)
constexpr int kBwdDqKeys = 64;    // keys per dQ K/V tile
constexpr int kBwdPoolCounters = 16;  // single-pass backward: 8 task pools, a done count, padding

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_fwd_dropout(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_fwd_poly(const FwdArgs& a, int d, hipStream_t s);
constexpr int kFwdMaxPools = 8;          // persistent forward: task queues (one per XCD)
constexpr int kFwdPoolCounters = 16;     // its counters: the queues, the leaver count, padding
hipError_t launch_fwd_persistent(FwdArgs a, int d, hipStream_t s);
hipError_t launch_exp2_poly(const float* x, float* y, long n, hipStream_t s);
hipError_t launch_bwd_dropout(const BwdArgs& a, int d, hipStream_t s);
constexpr int kFp8Block = 64;     // rows per FP8 quantisation block (one scale each)
hipError_t launch_quantize_fp8(const void* x, const float* signs, void* x8, float* scales, int B, int N, int H,
                               int d, hipStream_t s);
hipError_t launch_decode(const DecArgs& a, hipStream_t s);
// Device address of the static decode scratch array (kDecScratchBytes) on the current device;
// looked up once per device.
hipError_t decode_scratch(void** ptr);
hipError_t launch_bwd(const BwdArgs& a, int d, hipStream_t s);
// The single-pass backward (d = 128): all five products in one key-block-outer pass, dQ summed in
// the workspace in a fixed order. Supported shapes: bwd_single_pass_supported.
bool bwd_single_pass_supported(const BwdArgs& a, int d);
hipError_t launch_bwd_single_pass(const BwdArgs& a, int d, hipStream_t s);

}  // namespace fa
