// Top-k weighted combine / unpermute, plus the optional shared-expert term.
//
// Combine of the k expert outputs of a token: DisagMoE technical summary,
// "2.2 AF-Pipe".  Bound by HBM: each output row reads its k expert rows
// once (16-byte vectors) and is written once.  The k terms are added in
// slot order, so the result is deterministic.
//
// One workgroup per token.  The token's k rows and weights are read once
// (scalar loads); k is a template parameter so each thread keeps all k
// row loads of two 16-byte chunks in flight before it adds them.  The rows
// come as fp32 (combine_kernel) or in the compact fp16 form layer 1 writes
// on the default path (combine_f16_kernel, half the bytes).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;  // 16-byte chunks per thread in flight

// KS = k (1..8), or 0: no routed term (inv == NULL)
template <int KS>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const f32x4* __restrict__ y_perm, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, int vecs, const f32x4* __restrict__ y_shared,
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
    const float* __restrict__ topk_w, int vecs, int k, const f32x4* __restrict__ y_shared,
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
                     reinterpret_cast<const f32x4*>(y_perm), inv, topk_w, d / 4,
                     reinterpret_cast<const f32x4*>(y_shared), gate_logit, accumulate ? 1 : 0,
                     reinterpret_cast<f32x4*>(y));
}

// ---- compact rows (layer 1's fp16 output): 8 fp16 values per 16-byte
// chunk and one restoring factor per 32-column row segment (4 chunks), so
// that y_perm[r, c] = y_h[r, c] * y_s[r, c / 32] exactly.  The factor is a
// power of two, so w * factor is exact and each term w * factor * h equals
// w * y_perm[r, c] as the fp32 combine forms it: both combines give the
// same bits for the same rows.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void add_f16_chunk(f32x4& lo, f32x4& hi, float c, u32x4 raw) {
  const f16x8 h = __builtin_bit_cast(f16x8, raw);
  lo += c * f32x4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]),
                  static_cast<float>(h[3])};
  hi += c * f32x4{static_cast<float>(h[4]), static_cast<float>(h[5]), static_cast<float>(h[6]),
                  static_cast<float>(h[7])};
}

// KS = k (1..8), or 0: no routed term (inv == NULL).  chunks = d / 8,
// segs = d / 32; y is written as two 16-byte vectors per chunk.
template <int KS>
__global__ __launch_bounds__(kThreads) void combine_f16_kernel(
    const u32x4* __restrict__ y_h, const float* __restrict__ y_s, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, int chunks, const u32x4* __restrict__ ys_h,
    const float* __restrict__ ys_s, const float* __restrict__ gate_logit, int accumulate,
    f32x4* __restrict__ y) {
  const int t = blockIdx.x;
  const int segs = chunks >> 2;
  float g = 1.f;
  if (ys_h && gate_logit) g = 1.f / (1.f + __expf(-gate_logit[t]));
  int r[KS > 0 ? KS : 1];
  float w[KS > 0 ? KS : 1];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    r[j] = inv[(size_t)t * KS + j];
    w[j] = topk_w[(size_t)t * KS + j];
  }
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const u32x4 zero_u = {0u, 0u, 0u, 0u};
  f32x4* yt = y + (size_t)t * chunks * 2;
  for (int c0 = threadIdx.x; c0 < chunks; c0 += kThreads * kUnroll) {
    u32x4 src[kUnroll][KS > 0 ? KS : 1];
    float fac[kUnroll][KS > 0 ? KS : 1];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kThreads;
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        src[u][j] = c < chunks ? __builtin_nontemporal_load(y_h + (size_t)r[j] * chunks + c) : zero_u;
        fac[u][j] = c < chunks ? y_s[(size_t)r[j] * segs + (c >> 2)] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kThreads;
      if (c >= chunks) break;
      f32x4 lo = zero, hi = zero;
#pragma unroll
      for (int j = 0; j < KS; ++j) add_f16_chunk(lo, hi, w[j] * fac[u][j], src[u][j]);
      if (ys_h)
        add_f16_chunk(lo, hi, g * ys_s[(size_t)t * segs + (c >> 2)],
                      __builtin_nontemporal_load(ys_h + (size_t)t * chunks + c));
      const f32x4 a0 = accumulate ? yt[2 * c] : zero;
      const f32x4 a1 = accumulate ? yt[2 * c + 1] : zero;
      yt[2 * c] = a0 + lo;
      yt[2 * c + 1] = a1 + hi;
    }
  }
}

// any k: slot loop at run time
__global__ __launch_bounds__(kThreads) void combine_f16_any_kernel(
    const u32x4* __restrict__ y_h, const float* __restrict__ y_s, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, int chunks, int k, const u32x4* __restrict__ ys_h,
    const float* __restrict__ ys_s, const float* __restrict__ gate_logit, int accumulate,
    f32x4* __restrict__ y) {
  const int t = blockIdx.x;
  const int segs = chunks >> 2;
  float g = 1.f;
  if (ys_h && gate_logit) g = 1.f / (1.f + __expf(-gate_logit[t]));
  f32x4* yt = y + (size_t)t * chunks * 2;
  for (int c = threadIdx.x; c < chunks; c += kThreads) {
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
    for (int j = 0; j < k; ++j) {
      const int r = inv[(size_t)t * k + j];
      add_f16_chunk(lo, hi, topk_w[(size_t)t * k + j] * y_s[(size_t)r * segs + (c >> 2)],
                    y_h[(size_t)r * chunks + c]);
    }
    if (ys_h) add_f16_chunk(lo, hi, g * ys_s[(size_t)t * segs + (c >> 2)], ys_h[(size_t)t * chunks + c]);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 a0 = accumulate ? yt[2 * c] : zero;
    const f32x4 a1 = accumulate ? yt[2 * c + 1] : zero;
    yt[2 * c] = a0 + lo;
    yt[2 * c + 1] = a1 + hi;
  }
}

template <int KS>
void launch_f16_k(const uint16_t* y_h, const float* y_s, const int32_t* inv, const float* topk_w,
                  int T, int d, const uint16_t* ys_h, const float* ys_s, const float* gate_logit,
                  bool accumulate, float* y, hipStream_t s) {
  hipLaunchKernelGGL((combine_f16_kernel<KS>), dim3(T), dim3(kThreads), 0, s,
                     reinterpret_cast<const u32x4*>(y_h), y_s, inv, topk_w, d / 8,
                     reinterpret_cast<const u32x4*>(ys_h), ys_s, gate_logit, accumulate ? 1 : 0,
                     reinterpret_cast<f32x4*>(y));
}

}  // namespace

hipError_t launch_combine_f16(const uint16_t* y_h, const float* y_s, const int32_t* inv,
                              const float* topk_w, int T, int d, int k, const uint16_t* ys_h,
                              const float* ys_s, const float* gate_logit, bool accumulate,
                              float* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
#define MOE_F16_K(KS) \
  launch_f16_k<KS>(y_h, y_s, inv, topk_w, T, d, ys_h, ys_s, gate_logit, accumulate, y, s)
  switch (inv ? k : 0) {
    case 0: MOE_F16_K(0); break;
    case 1: MOE_F16_K(1); break;
    case 2: MOE_F16_K(2); break;
    case 3: MOE_F16_K(3); break;
    case 4: MOE_F16_K(4); break;
    case 5: MOE_F16_K(5); break;
    case 6: MOE_F16_K(6); break;
    case 7: MOE_F16_K(7); break;
    case 8: MOE_F16_K(8); break;
    default:
      hipLaunchKernelGGL(combine_f16_any_kernel, dim3(T), dim3(kThreads), 0, s,
                         reinterpret_cast<const u32x4*>(y_h), y_s, inv, topk_w, d / 8, k,
                         reinterpret_cast<const u32x4*>(ys_h), ys_s, gate_logit,
                         accumulate ? 1 : 0, reinterpret_cast<f32x4*>(y));
  }
#undef MOE_F16_K
  return hipGetLastError();
}

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
                         reinterpret_cast<const f32x4*>(y_perm), inv, topk_w, d / 4, k,
                         reinterpret_cast<const f32x4*>(y_shared), gate_logit, accumulate ? 1 : 0,
                         reinterpret_cast<f32x4*>(y));
  }
  return hipGetLastError();
}

}  // namespace moe
