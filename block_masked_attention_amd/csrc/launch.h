// Kernel launchers shared by the C ABI (api.cpp) and the kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace bdattn {

struct FwdArgs {
  const void *q_c, *k_c, *v_c, *q_x, *k_x, *v_x;
  void *o_c, *o_x;
  float *lse_c, *lse_x;
  const int32_t* ids;      // device: global id of each local corrupted block
  const BdDocSpan* docs;   // device: document of each global block, or nullptr
  const int32_t* kv_map;   // device: buffer tile of each clean key tile, or nullptr
  int32_t n_kv_map;
  const FwdItem* items;    // device work list
  int32_t n_items;
  int32_t* claim;          // kClaimQueues work-claim counters, or nullptr: workgroup i runs item i
  int32_t persist;         // > 0: a grid of `persist` workgroups that claim items until none is left
  int32_t B, H, Hkv, Gw, rows_per_item;
  int32_t n_clean_q, clean_q_start, n_clean_kv, n_corr;
  int32_t token_causal;    // clean rows see their own block up to their position only
  int32_t clean_kv_start;  // global position of clean buffer row 0
  int32_t corr_keys;       // the local corrupted keys are present
  int32_t precision;       // bdattn_precision: float32 O (>= 1), split P (2)
  float scale_log2;        // softmax scale * log2(e)
};

struct BwdArgs {
  const void *q_c, *k_c, *v_c, *q_x, *k_x, *v_x;
  const void *o_c, *o_x, *do_c, *do_x;
  const float *lse_c, *lse_x;
  void *dq_c, *dq_x, *dk_c, *dv_c, *dk_x, *dv_x;
  const int32_t* ids;
  const BdDocSpan* docs;   // device: document of each global block, or nullptr
  const int32_t* kv_map;   // device: buffer tile of each clean key tile, or nullptr
  int32_t n_kv_map;
  const FwdItem* q_items;  // dQ kernel: the forward's query-tile work list
  int32_t n_q_items;
  const BwdItem* kv_items;  // dK/dV kernel: key-tile work list
  int32_t n_kv_items;
  int32_t *claim_q, *claim_kv;  // work-claim counters of the two lists, or nullptr (static)
  int32_t persist;         // dQ kernel: > 0, a grid of `persist` workgroups that claim items until none is left
  float *d_c, *d_x;        // workspace: -D = -rowsum(dO * O)    [H][row_pad(n)]
  float *l2_c, *l2_x;      // workspace: LSE * log2(e), +inf pad [H][row_pad(n)]
  int32_t B, H, Hkv, Gw, rows_per_item;
  int32_t n_clean_q, clean_q_start, n_clean_kv, n_corr;
  int32_t token_causal;    // clean rows see their own block up to their position only
  int32_t clean_kv_start;  // global position of clean buffer row 0
  int32_t corr_keys;       // the local corrupted keys are present
  int32_t precision;       // bdattn_precision: float32 O (read), dQ, dK, dV (>= 1), split P, dS (2)
  float scale, scale_log2;
};

// Records `msg` as the calling thread's last error (bdattn_last_error) and
// returns `status`.
int record_error(int status, const std::string& msg);

// True if this build has kernels for (dtype, d).
bool have_kernels(int dtype, int d);

// Events recorded around the main kernels (ev == nullptr: none). The forward
// records ev[0] around its kernel; the backward records ev[0] around the dQ
// kernel and ev[1] around the dK/dV kernel.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Benchmark instrumentation (bdattn_profile_enable): kernel slots 0 forward,
// 1 backward dQ, 2 backward dK/dV, then the linear cross-entropy's 3 logits
// product, 4 row kernel, 5 dH product, 6 dW product. profile_events fills
// ev[0..n-1] with fresh events for slots first..first+n-1 and returns ev, or
// returns nullptr when profiling is off; every returned pair must be recorded.
constexpr int kProfiledKernels = 7;
const KernelEvents* profile_events(int first, int n, KernelEvents* ev);

hipError_t launch_fwd(const FwdArgs& a, int dtype, int d, hipStream_t stream,
                      const KernelEvents* ev);
hipError_t launch_bwd(const BwdArgs& a, int dtype, int d, hipStream_t stream,
                      const KernelEvents* ev);
// The key-tile dK/dV kernel alone (called by launch_bwd after the dQ kernel).
hipError_t launch_dkdv(const BwdArgs& a, int dtype, int d, hipStream_t stream);
// Measured alternatives (kernels_bwd_fused.hip): dK/dV with one wave per 32
// keys in both roles, and the whole backward in one kernel with dQ by float
// atomics (bf16, d = 128, contiguous clean K/V: bwd_fused_supported).
hipError_t launch_dkdv_fused(const BwdArgs& a, int dtype, int d, hipStream_t stream);
bool bwd_fused_supported(const BwdArgs& a, int dtype, int d);
hipError_t launch_bwd_fused(const BwdArgs& a, int dtype, int d, hipStream_t stream);
// Merge of two partial results (bdattn_merge).
hipError_t launch_merge(int64_t n_rows, int H, int d, int dtype, const void* o_a,
                        const float* lse_a, const void* o_b, const float* lse_b, void* o,
                        float* lse, hipStream_t stream);

}  // namespace bdattn
