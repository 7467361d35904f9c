// Top-k weighted combine / unpermute, plus the optional shared-expert term.
//
// Combine of the k expert outputs of a token: DisagMoE technical summary,
// "2.2 AF-Pipe".  Bound by HBM: each output row reads its k expert rows
// once (16-byte vectors) and is written once.  The k terms are added in
// slot order, so the result is deterministic.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const f32x4* __restrict__ y_perm, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, int T, int vecs, int k, const f32x4* __restrict__ y_shared,
    const float* __restrict__ gate_logit, int accumulate, f32x4* __restrict__ y) {
  const int t = blockIdx.x;
  float g = 1.f;
  if (y_shared && gate_logit) g = 1.f / (1.f + __expf(-gate_logit[t]));
  for (int c = threadIdx.x; c < vecs; c += kThreads) {
    f32x4 acc = accumulate ? y[(size_t)t * vecs + c] : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; inv && j < k; ++j) {
      const int r = inv[(size_t)t * k + j];
      const float w = topk_w[(size_t)t * k + j];
      const f32x4 src = y_perm[(size_t)r * vecs + c];
      v += w * src;
    }
    if (y_shared) v += g * y_shared[(size_t)t * vecs + c];
    y[(size_t)t * vecs + c] = acc + v;
  }
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* inv, const float* topk_w, int T,
                          int d, int k, const float* y_shared, const float* gate_logit,
                          bool accumulate, float* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(kThreads), 0, s,
                     reinterpret_cast<const f32x4*>(y_perm), inv, topk_w, T, d / 4, k,
                     reinterpret_cast<const f32x4*>(y_shared), gate_logit, accumulate ? 1 : 0,
                     reinterpret_cast<f32x4*>(y));
  return hipGetLastError();
}

}  // namespace moe
