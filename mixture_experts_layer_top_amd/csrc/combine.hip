// Top-k weighted combine / unpermute, plus the optional shared-expert term.
//
// Combine of the k expert outputs of a token: DisagMoE technical summary,
// "2.2 AF-Pipe".  Bound by HBM: each output row reads its k expert rows
// once (16-byte vectors) and is written once.  The k terms are added in
// slot order, so the result is deterministic.
//
// One workgroup per token.  The token's k rows and weights are read once
// (scalar loads); k is a template parameter so each thread keeps all k
// row loads of two 16-byte chunks in flight before it adds them.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;  // 16-byte chunks per thread in flight

// KS = k (1..8), or 0: no routed term (inv == NULL)
template <int KS>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const f32x4* __restrict__ y_perm, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, int T, int vecs, const f32x4* __restrict__ y_shared,
    const float* __restrict__ gate_logit, int accumulate, f32x4* __restrict__ y) {
  const int t = blockIdx.x;
  float g = 1.f;
  if (y_shared && gate_logit) g = 1.f / (1.f + __expf(-gate_logit[t]));
  int r[KS > 0 ? KS : 1];
  float w[KS > 0 ? KS : 1];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    r[j] = inv[(size_t)t * KS + j];
    w[j] = topk_w[(size_t)t * KS + j];
  }
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4* yt = y + (size_t)t * vecs;
  const f32x4* st = y_shared ? y_shared + (size_t)t * vecs : nullptr;
  for (int c0 = threadIdx.x; c0 < vecs; c0 += kThreads * kUnroll) {
    f32x4 src[kUnroll][KS > 0 ? KS : 1];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kThreads;
#pragma unroll
      for (int j = 0; j < KS; ++j)
        src[u][j] = c < vecs ? __builtin_nontemporal_load(y_perm + (size_t)r[j] * vecs + c) : zero;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kThreads;
      if (c >= vecs) break;
      f32x4 v = zero;
#pragma unroll
      for (int j = 0; j < KS; ++j) v += w[j] * src[u][j];
      if (st) v += g * st[c];
      const f32x4 acc = accumulate ? yt[c] : zero;
      yt[c] = acc + v;
    }
  }
}

// any k (the C ABI allows up to 256): slot loop at run time
__global__ __launch_bounds__(kThreads) void combine_any_kernel(
    const f32x4* __restrict__ y_perm, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, int T, int vecs, int k, const f32x4* __restrict__ y_shared,
    const float* __restrict__ gate_logit, int accumulate, f32x4* __restrict__ y) {
  const int t = blockIdx.x;
  float g = 1.f;
  if (y_shared && gate_logit) g = 1.f / (1.f + __expf(-gate_logit[t]));
  for (int c = threadIdx.x; c < vecs; c += kThreads) {
    f32x4 acc = accumulate ? y[(size_t)t * vecs + c] : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int r = inv[(size_t)t * k + j];
      v += topk_w[(size_t)t * k + j] * y_perm[(size_t)r * vecs + c];
    }
    if (y_shared) v += g * y_shared[(size_t)t * vecs + c];
    y[(size_t)t * vecs + c] = acc + v;
  }
}

template <int KS>
void launch_k(const float* y_perm, const int32_t* inv, const float* topk_w, int T, int d,
              const float* y_shared, const float* gate_logit, bool accumulate, float* y,
              hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<KS>), dim3(T), dim3(kThreads), 0, s,
                     reinterpret_cast<const f32x4*>(y_perm), inv, topk_w, T, d / 4,
                     reinterpret_cast<const f32x4*>(y_shared), gate_logit, accumulate ? 1 : 0,
                     reinterpret_cast<f32x4*>(y));
}

}  // namespace

hipError_t launch_combine(const float* y_perm, const int32_t* inv, const float* topk_w, int T,
                          int d, int k, const float* y_shared, const float* gate_logit,
                          bool accumulate, float* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  switch (inv ? k : 0) {
    case 0: launch_k<0>(y_perm, inv, topk_w, T, d, y_shared, gate_logit, accumulate, y, s); break;
    case 1: launch_k<1>(y_perm, inv, topk_w, T, d, y_shared, gate_logit, accumulate, y, s); break;
    case 2: launch_k<2>(y_perm, inv, topk_w, T, d, y_shared, gate_logit, accumulate, y, s); break;
    case 3: launch_k<3>(y_perm, inv, topk_w, T, d, y_shared, gate_logit, accumulate, y, s); break;
    case 4: launch_k<4>(y_perm, inv, topk_w, T, d, y_shared, gate_logit, accumulate, y, s); break;
    case 5: launch_k<5>(y_perm, inv, topk_w, T, d, y_shared, gate_logit, accumulate, y, s); break;
    case 6: launch_k<6>(y_perm, inv, topk_w, T, d, y_shared, gate_logit, accumulate, y, s); break;
    case 7: launch_k<7>(y_perm, inv, topk_w, T, d, y_shared, gate_logit, accumulate, y, s); break;
    case 8: launch_k<8>(y_perm, inv, topk_w, T, d, y_shared, gate_logit, accumulate, y, s); break;
    default:
      hipLaunchKernelGGL(combine_any_kernel, dim3(T), dim3(kThreads), 0, s,
                         reinterpret_cast<const f32x4*>(y_perm), inv, topk_w, T, d / 4, k,
                         reinterpret_cast<const f32x4*>(y_shared), gate_logit, accumulate ? 1 : 0,
                         reinterpret_cast<f32x4*>(y));
  }
  return hipGetLastError();
}

}  // namespace moe
