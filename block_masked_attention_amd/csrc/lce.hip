// Token-chunked linear cross-entropy (include/bdattn_lce.h): the vocabulary
// projections by rocBLAS, chunk of tokens by chunk of tokens, and the fused
// softmax / cross-entropy kernels of gfx950 that turn each chunk's logits
// into the loss, the log-sum-exp and the bf16 logit gradient ("Block
// Parallelism for Efficient Distributed Long-Context Diffusion Language Model
// Training", §5.1, Experimental setup: library projections plus fused
// softmax/CE kernels, no full-sequence logits).
//
// The row kernels are bound by HBM: each reads a row of V float32 logits once
// (the fused forward+backward kernel twice: the second read mostly hits the
// last-level cache) and writes V bf16 gradients. One workgroup of 256 threads
// per token row, 16-byte loads: a row of V = 131,072 logits is 128 loads per
// thread. The softmax statistics are an online (max, sum of exp2) pair per
// thread in base 2, merged across the wave by shuffles and across the four
// waves through LDS.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <unordered_map>

#include "../../include/bdattn.h"
#include "../../include/bdattn_lce.h"
#include "launch.h"

namespace bdattn {
namespace {

constexpr int kRowThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

__device__ __forceinline__ uint32_t bf16_bits(float f) {  // round to nearest even
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct MaxSum {
  float m, s;  // running maximum and sum of exp2(y - m), base-2 units
};

__device__ __forceinline__ MaxSum ms_merge(MaxSum a, MaxSum b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -__builtin_inff()) return {m, 0.f};
  return {m, a.s * exp2f(a.m - m) + b.s * exp2f(b.m - m)};
}

// (max, sum) of one row of V float32 logits in base 2, identical on every
// thread of the workgroup afterwards.
__device__ MaxSum row_max_sum(const float4* row4, int n4) {
  MaxSum t{-__builtin_inff(), 0.f};
  for (int k = threadIdx.x; k < n4; k += kRowThreads) {
    const float4 x = row4[k];
    const float y0 = x.x * kLog2e, y1 = x.y * kLog2e, y2 = x.z * kLog2e, y3 = x.w * kLog2e;
    const float m4 = fmaxf(fmaxf(y0, y1), fmaxf(y2, y3));
    if (m4 > t.m) {
      t.s = t.m == -__builtin_inff() ? 0.f : t.s * exp2f(t.m - m4);
      t.m = m4;
    }
    t.s += exp2f(y0 - t.m) + exp2f(y1 - t.m) + exp2f(y2 - t.m) + exp2f(y3 - t.m);
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    MaxSum o{__shfl_xor(t.m, w), __shfl_xor(t.s, w)};
    t = ms_merge(t, o);
  }
  __shared__ MaxSum part[kRowThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = t;
  __syncthreads();
  MaxSum r = part[0];
#pragma unroll
  for (int i = 1; i < kRowThreads / 64; ++i) r = ms_merge(r, part[i]);
  return r;
}

// LSE and loss of each token row of a chunk.
__global__ __launch_bounds__(kRowThreads) void lce_loss_kernel(const float* logits, int V,
                                                               const int32_t* targets,
                                                               int ignore, float* loss,
                                                               float* lse) {
  const int64_t i = blockIdx.x;
  const float* row = logits + i * V;
  const MaxSum r = row_max_sum((const float4*)row, V / 4);
  if (threadIdx.x == 0) {
    const float l = (r.m + log2f(r.s)) * kLn2;
    const int t = targets[i];
    lse[i] = l;
    // (a target outside [0, V) reads no logit: its loss is NaN)
    loss[i] = t == ignore ? 0.f : (t >= 0 && t < V ? l - row[t] : __builtin_nanf(""));
  }
}

// G = g (softmax - onehot) of one row, rounded to bf16, from the row's LSE
// (base 2: lse2 = LSE log2 e).
__device__ __forceinline__ void write_grad(const float4* row4, int n4, uint2* out4, float lse2,
                                           float g, int t) {
  for (int k = threadIdx.x; k < n4; k += kRowThreads) {
    const float4 x = row4[k];
    float p0 = exp2f(fmaf(x.x, kLog2e, -lse2)) * g, p1 = exp2f(fmaf(x.y, kLog2e, -lse2)) * g;
    float p2 = exp2f(fmaf(x.z, kLog2e, -lse2)) * g, p3 = exp2f(fmaf(x.w, kLog2e, -lse2)) * g;
    const int j = 4 * k;
    if (t - j >= 0 && t - j < 4) {
      if (t == j) p0 -= g;
      else if (t == j + 1) p1 -= g;
      else if (t == j + 2) p2 -= g;
      else p3 -= g;
    }
    out4[k] = make_uint2(bf16_bits(p0) | (bf16_bits(p1) << 16), bf16_bits(p2) | (bf16_bits(p3) << 16));
  }
}

// The logit gradient of each token row of a chunk, from the forward's LSE.
__global__ __launch_bounds__(kRowThreads) void lce_grad_kernel(const float* logits, int V,
                                                               const int32_t* targets,
                                                               int ignore, const float* lse,
                                                               const float* dloss,
                                                               uint16_t* grad) {
  const int64_t i = blockIdx.x;
  const int t = targets[i];
  const float g = t == ignore ? 0.f : dloss[i];
  write_grad((const float4*)(logits + i * V), V / 4, (uint2*)(grad + i * V), lse[i] * kLog2e, g,
             t == ignore ? -1 : t);
}

// Forward and backward of each token row of a chunk in one kernel.
__global__ __launch_bounds__(kRowThreads) void lce_fused_kernel(const float* logits, int V,
                                                                const int32_t* targets,
                                                                int ignore, const float* dloss,
                                                                float* loss, float* lse,
                                                                uint16_t* grad) {
  const int64_t i = blockIdx.x;
  const float* row = logits + i * V;
  const MaxSum r = row_max_sum((const float4*)row, V / 4);
  // the gradient uses the stored LSE, as the separate backward does, so the
  // two paths give bitwise equal results
  const float l = (r.m + log2f(r.s)) * kLn2;
  const float lse2 = l * kLog2e;
  const int t = targets[i];
  if (threadIdx.x == 0) {
    lse[i] = l;
    loss[i] = t == ignore ? 0.f : (t >= 0 && t < V ? l - row[t] : __builtin_nanf(""));
  }
  const float g = t == ignore ? 0.f : dloss[i];
  write_grad((const float4*)row, V / 4, (uint2*)(grad + i * V), lse2, g, t == ignore ? -1 : t);
}

__global__ void fill_zero_kernel(float4* p, int64_t n4) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n4) p[k] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ------------------------------------------------------------------ host
struct Shape {
  int64_t N;
  int32_t D, V, C, ignore;
};

int check_problem(const bdattn_lce_problem* p, Shape* s) {
  if (!p) return record_error(BDATTN_ERR_INVALID_ARG, "problem descriptor is NULL");
  if (p->n_tokens < 0 || p->hidden < 8 || p->hidden % 8 || p->vocab < 8 || p->vocab % 8 ||
      p->chunk < 1)
    return record_error(BDATTN_ERR_SHAPE,
                        "need n_tokens >= 0, hidden and vocab multiples of 8 (>= 8), chunk >= 1");
  if (int64_t(p->chunk) * p->vocab >= (int64_t(1) << 31))
    return record_error(BDATTN_ERR_SHAPE, "chunk * vocab must stay below 2^31");
  if (p->n_tokens >= (int64_t(1) << 31))
    return record_error(BDATTN_ERR_SHAPE, "n_tokens must stay below 2^31");
  s->N = p->n_tokens;
  s->D = p->hidden;
  s->V = p->vocab;
  s->C = int32_t(std::min<int64_t>(p->chunk, std::max<int64_t>(1, p->n_tokens)));
  s->ignore = p->ignore_index;
  return BDATTN_OK;
}

size_t ws_bytes(const Shape& s, int pass) {
  const size_t rows = size_t(s.C) * size_t(s.V);
  return align_up(rows * sizeof(float)) + (pass ? align_up(rows * sizeof(uint16_t)) : 0);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_ptr(const void* p, int64_t n, uintptr_t a, const char* name) {
  if (n == 0) return BDATTN_OK;
  if (!p) return record_error(BDATTN_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned(p, a)) return record_error(BDATTN_ERR_INVALID_ARG, std::string(name) + " is misaligned");
  return BDATTN_OK;
}

// One rocBLAS handle per (thread, device), bound to the call's stream.
int blas_handle(hipStream_t s, rocblas_handle* out) {
  thread_local std::unordered_map<int, rocblas_handle> handles;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return record_error(BDATTN_ERR_HIP, "hipGetDevice failed");
  rocblas_handle& h = handles[dev];
  if (!h) {
    if (rocblas_create_handle(&h) != rocblas_status_success) {
      h = nullptr;
      return record_error(BDATTN_ERR_HIP, "rocblas_create_handle failed");
    }
    // products without atomics: every result is reproducible
    (void)rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed);
  }
  if (rocblas_set_stream(h, s) != rocblas_status_success)
    return record_error(BDATTN_ERR_HIP, "rocblas_set_stream failed");
  *out = h;
  return BDATTN_OK;
}

// Column-major product D = alpha op(A) op(B) + beta C with bf16 operands and
// fp32 accumulation; `out_bf16` selects the type of C = D.
int gemm(rocblas_handle h, rocblas_operation ta, rocblas_operation tb, int m, int n, int k,
         const void* a, int lda, const void* b, int ldb, float beta, void* c, int ldc,
         bool out_bf16, const char* what) {
  const float alpha = 1.f;
  const rocblas_datatype ct = out_bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  rocblas_status st = rocblas_gemm_ex(h, ta, tb, m, n, k, &alpha, a, rocblas_datatype_bf16_r, lda,
                                      b, rocblas_datatype_bf16_r, ldb, &beta, c, ct, ldc, c, ct,
                                      ldc, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success)
    return record_error(BDATTN_ERR_HIP, std::string("rocblas_gemm_ex (") + what + "): " +
                                            rocblas_status_to_string(st));
  return BDATTN_OK;
}

enum Mode { kFwd, kBwd, kFwdBwd };

int run(Mode mode, const bdattn_lce_problem* p, const void* h_, const void* w_,
        const int32_t* targets, const float* lse_in, const float* dloss, float* loss, float* lse,
        void* dh_, float* dw, void* workspace, size_t ws_size, void* stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st) return st;
  const int64_t nh = s.N * s.D, nw = int64_t(s.V) * s.D;
  if ((st = check_ptr(h_, nh, 16, "h")) || (st = check_ptr(w_, nw, 16, "w")) ||
      (st = check_ptr(targets, s.N, 4, "targets")))
    return st;
  if (mode != kBwd && ((st = check_ptr(loss, s.N, 4, "loss")) || (st = check_ptr(lse, s.N, 4, "lse"))))
    return st;
  if (mode == kBwd && (st = check_ptr(lse_in, s.N, 4, "lse"))) return st;
  if (mode != kFwd && ((st = check_ptr(dloss, s.N, 4, "dloss")) || (st = check_ptr(dh_, nh, 16, "dh")) ||
                       (st = check_ptr(dw, nw, 16, "dw"))))
    return st;
  const size_t need = ws_bytes(s, mode == kFwd ? 0 : 1);
  if (s.N > 0 && (!workspace || !aligned(workspace, kAlign) || ws_size < need))
    return record_error(BDATTN_ERR_WORKSPACE, "workspace missing, misaligned or smaller than " +
                                                  std::to_string(need) + " bytes");
  hipStream_t hs = (hipStream_t)stream;
  if (s.N == 0) {  // no token: dW is zero
    if (mode != kFwd && nw > 0)
      hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned((nw / 4 + 255) / 256)), dim3(256), 0, hs,
                         (float4*)dw, nw / 4);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? BDATTN_OK : record_error(BDATTN_ERR_HIP, hipGetErrorString(e));
  }
  rocblas_handle bh;
  if ((st = blas_handle(hs, &bh))) return st;
  const uint16_t* h = (const uint16_t*)h_;
  const uint16_t* w = (const uint16_t*)w_;
  uint16_t* dh = (uint16_t*)dh_;
  float* logits = (float*)workspace;
  uint16_t* grad = (uint16_t*)((char*)workspace + align_up(size_t(s.C) * s.V * sizeof(float)));
  for (int64_t r0 = 0; r0 < s.N; r0 += s.C) {
    const int cc = int(std::min<int64_t>(s.C, s.N - r0));
    // benchmark events (slots 3..6: logits, row kernel, dH, dW), if profiling
    KernelEvents evs[4];
    const KernelEvents* ev = profile_events(3, mode == kFwd ? 2 : 4, evs);
    auto mark = [&](int k, bool stop) {
      if (ev) (void)hipEventRecord(stop ? ev[k].stop : ev[k].start, hs);
    };
    // logits [cc, V] = h[r0:r0+cc] w^T   (column-major: [V, cc] = w^T' h')
    mark(0, false);
    if ((st = gemm(bh, rocblas_operation_transpose, rocblas_operation_none, s.V, cc, s.D, w, s.D,
                   h + r0 * s.D, s.D, 0.f, logits, s.V, false, "logits")))
      return st;
    mark(0, true);
    mark(1, false);
    if (mode == kFwd)
      hipLaunchKernelGGL(lce_loss_kernel, dim3(cc), dim3(kRowThreads), 0, hs, logits, s.V,
                         targets + r0, s.ignore, loss + r0, lse + r0);
    else if (mode == kBwd)
      hipLaunchKernelGGL(lce_grad_kernel, dim3(cc), dim3(kRowThreads), 0, hs, logits, s.V,
                         targets + r0, s.ignore, lse_in + r0, dloss + r0, grad);
    else
      hipLaunchKernelGGL(lce_fused_kernel, dim3(cc), dim3(kRowThreads), 0, hs, logits, s.V,
                         targets + r0, s.ignore, dloss + r0, loss + r0, lse + r0, grad);
    mark(1, true);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return record_error(BDATTN_ERR_HIP, std::string("row kernel: ") + hipGetErrorString(e));
    if (mode == kFwd) continue;
    // dh[r0:r0+cc] = G w   (column-major: [D, cc] = w' G')
    mark(2, false);
    if ((st = gemm(bh, rocblas_operation_none, rocblas_operation_none, s.D, cc, s.V, w, s.D, grad,
                   s.V, 0.f, dh + r0 * s.D, s.D, true, "dh")))
      return st;
    mark(2, true);
    // dw (+)= G^T h[r0:r0+cc]   (column-major: [D, V] (+)= h' G'^T)
    mark(3, false);
    if ((st = gemm(bh, rocblas_operation_none, rocblas_operation_transpose, s.D, s.V, cc,
                   h + r0 * s.D, s.D, grad, s.V, r0 == 0 ? 0.f : 1.f, dw, s.D, false, "dw")))
      return st;
    mark(3, true);
  }
  return BDATTN_OK;
}

}  // namespace
}  // namespace bdattn

extern "C" {

int bdattn_lce_workspace_size(const bdattn_lce_problem* p, int pass, size_t* bytes) {
  if (!bytes) return bdattn::record_error(BDATTN_ERR_INVALID_ARG, "bytes is NULL");
  if (pass != 0 && pass != 1) return bdattn::record_error(BDATTN_ERR_INVALID_ARG, "pass must be 0 or 1");
  bdattn::Shape s;
  int st = bdattn::check_problem(p, &s);
  if (st) return st;
  *bytes = bdattn::ws_bytes(s, pass);
  return BDATTN_OK;
}

int bdattn_lce_fwd(const bdattn_lce_problem* p, const void* h, const void* w,
                   const int32_t* targets, float* loss, float* lse, void* workspace,
                   size_t ws_bytes, void* hip_stream) {
  return bdattn::run(bdattn::kFwd, p, h, w, targets, nullptr, nullptr, loss, lse, nullptr, nullptr,
                     workspace, ws_bytes, hip_stream);
}

int bdattn_lce_bwd(const bdattn_lce_problem* p, const void* h, const void* w,
                   const int32_t* targets, const float* lse, const float* dloss, void* dh,
                   float* dw, void* workspace, size_t ws_bytes, void* hip_stream) {
  return bdattn::run(bdattn::kBwd, p, h, w, targets, lse, dloss, nullptr, nullptr, dh, dw,
                     workspace, ws_bytes, hip_stream);
}

int bdattn_lce_fwd_bwd(const bdattn_lce_problem* p, const void* h, const void* w,
                       const int32_t* targets, const float* dloss, float* loss, float* lse,
                       void* dh, float* dw, void* workspace, size_t ws_bytes, void* hip_stream) {
  return bdattn::run(bdattn::kFwdBwd, p, h, w, targets, nullptr, dloss, loss, lse, dh, dw,
                     workspace, ws_bytes, hip_stream);
}

}  // extern "C"
