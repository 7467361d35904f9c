// Router: logits, softmax top-k selection and weights, one pass over x.
//
// Top-k expert choice per token: DisagMoE technical summary, "2.2 AF-Pipe".
//
// bf16 path: a workgroup of 4 wave64s takes 64 tokens (16 per wave).  The
// logits L = x W_r are a skinny contraction (E <= 256 columns); each wave
// runs v_mfma_f32_16x16x32_bf16 with its 16 token rows as the A operand,
// read straight from HBM (16 contiguous bytes of K per lane), and W_r as the
// B operand.  W_r is row-major [d, E] (E contiguous), so a 64-row chunk of
// it is staged in LDS as is and read back with ds_read_b64_tr_b16, which
// hands each lane 4 consecutive K values of one column.  Products of bf16
// are exact in fp32; the sum is fp32.  The kernel is bound by reading x
// from HBM once.
//
// Selection and weights: the logits go to LDS; 4 lanes serve one token and
// each scans every 4th expert.  The j-th pick is the best (value desc,
// index asc) among experts strictly below the (j-1)-th pick in that order,
// so no pick is ever marked; equal logits go to the lower index.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTok = 64;   // tokens per workgroup
constexpr int kKC = 64;    // rows of W_r staged per chunk
constexpr int kThreads = 256;

struct RouteArgs {
  const void* x;
  const void* W;
  const float* bias;
  int T, d, E, k, renorm;
  int32_t* idx;
  float* w;
  float* logits_out;
};

// Softmax top-k over the logits rows of this workgroup (in LDS), one wave
// per 16 tokens, 4 lanes per token.
__device__ __forceinline__ void select_and_weigh(const float* ll, int lstride, const RouteArgs& a,
                                                 int t_base) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tt = wave * 16 + (lane >> 2);
  const int q = lane & 3;
  const int t = t_base + tt;
  const float* row = ll + tt * lstride;
  const int E = a.E, k = a.k;

  // full softmax denominator, relative to the row max
  float m = -INFINITY;
  for (int e = q; e < E; e += 4) m = fmaxf(m, row[e]);
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  float s = 0.f;
  for (int e = q; e < E; e += 4) s += __expf(row[e] - m);
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);

  // two passes of the same deterministic selection: first the sum over the
  // picks (renormalisation), then the outputs
  float sel_sum = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    float pv = INFINITY;
    int pe = -1;
    const float denom = a.renorm ? sel_sum : s;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
      for (int e = q; e < E; e += 4) {
        const float v = row[e];
        const bool below = (v < pv) || (v == pv && e > pe);
        const bool better = (v > bv) || (v == bv && e < be);
        if (below && better) {
          bv = v;
          be = e;
        }
      }
#pragma unroll
      for (int off = 1; off <= 2; off <<= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
      pv = bv;
      pe = be;
      const float ex = __expf(bv - m);
      if (pass == 0) {
        sel_sum += ex;
      } else if (q == 0 && t < a.T) {
        a.idx[(size_t)t * k + j] = be;
        a.w[(size_t)t * k + j] = ex / denom;
      }
    }
  }
}

__device__ __forceinline__ void write_logits(const float* ll, int lstride, const RouteArgs& a,
                                             int t_base) {
  if (a.logits_out == nullptr) return;
  const int n = kTok * a.E;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int tt = i / a.E, e = i - tt * a.E;
    const int t = t_base + tt;
    if (t < a.T) a.logits_out[(size_t)t * a.E + e] = ll[tt * lstride + e];
  }
}

// NB = ceil(E / 16) column blocks of 16 experts.
template <int NB>
__global__ __launch_bounds__(kThreads) void route_bf16_kernel(RouteArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int Ep = NB * 16;
  constexpr int ws = Ep + 8;  // LDS row stride of the W_r chunk, in bf16 (16 B pad)
  constexpr int ls = Ep + 1;  // LDS row stride of the logits, in floats
  bf16_t* wl = reinterpret_cast<bf16_t*>(smem);
  float* ll = reinterpret_cast<float*>(smem + kKC * ws * 2);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t_base = blockIdx.x * kTok;
  const int my_t = t_base + wave * 16 + (lane & 15);
  const bool t_ok = my_t < a.T;
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  const bf16_t* xrow = static_cast<const bf16_t*>(a.x) + (size_t)(t_ok ? my_t : 0) * a.d;
  const int d = a.d, E = a.E;

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < d; k0 += kKC) {
    __syncthreads();  // the previous chunk has been consumed
    for (int i = tid; i < kKC * Ep; i += kThreads) {
      const int r = i / Ep, c = i - r * Ep;
      bf16_t v = 0;
      if (k0 + r < d && c < E) v = W[(size_t)(k0 + r) * E + c];
      wl[r * ws + c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kKC; ks += 32) {
      const int kk = k0 + ks + (lane >> 4) * 8;
      bf16x8 av;
      if (t_ok && kk < d) {
        av = *reinterpret_cast<const bf16x8*>(xrow + kk);
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) av[u] = (__bf16)0.0f;
      }
      const int rr = ks + (lane >> 4) * 8 + ((lane & 15) >> 2);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int cc = nb * 16 + (lane & 3) * 4;
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
        const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(wl + rr * ws + cc));
        const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(wl + (rr + 4) * ws + cc));
        const bf16x8 bv = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nb], 0, 0, 0);
      }
    }
  }

  // accumulator lane layout of a 16x16 block: column = lane % 16, rows =
  // 4 * (lane / 16) + i
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int e = nb * 16 + (lane & 15);
    if (e < E) {
      const float b = a.bias ? a.bias[e] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = wave * 16 + (lane >> 4) * 4 + i;
        ll[tt * ls + e] = acc[nb][i] + b;
      }
    }
  }
  __syncthreads();
  write_logits(ll, ls, a, t_base);
  select_and_weigh(ll, ls, a, t_base);
}

// fp32 path (small layers): plain sequential FMA dot products.
__global__ __launch_bounds__(kThreads) void route_f32_kernel(RouteArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* ll = reinterpret_cast<float*>(smem);
  const int ls = a.E + 1;
  const int t_base = blockIdx.x * kTok;
  const float* x = static_cast<const float*>(a.x);
  const float* W = static_cast<const float*>(a.W);
  for (int i = threadIdx.x; i < kTok * a.E; i += kThreads) {
    const int tt = i / a.E, e = i - tt * a.E;
    const int t = t_base + tt;
    float acc = 0.f;
    if (t < a.T) {
      const float* xr = x + (size_t)t * a.d;
      for (int kk = 0; kk < a.d; ++kk) acc = fmaf(xr[kk], W[(size_t)kk * a.E + e], acc);
    }
    ll[tt * ls + e] = acc + (a.bias ? a.bias[e] : 0.f);
  }
  __syncthreads();
  write_logits(ll, ls, a, t_base);
  select_and_weigh(ll, ls, a, t_base);
}

template <int NB>
hipError_t launch_nb(const RouteArgs& a, int grid, hipStream_t s) {
  constexpr int Ep = NB * 16;
  const size_t lds = (size_t)kKC * (Ep + 8) * 2 + (size_t)kTok * (Ep + 1) * 4;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)route_bf16_kernel<NB>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(route_bf16_kernel<NB>, dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const void* x, const void* W_r, const float* bias, int T, int d, int E,
                        int k, bool renorm, bool bf16, int32_t* idx, float* w, float* logits_out,
                        hipStream_t s) {
  RouteArgs a{x, W_r, bias, T, d, E, k, renorm ? 1 : 0, idx, w, logits_out};
  const int grid = cdiv(T, kTok);
  if (!bf16) {
    const size_t lds = (size_t)kTok * (E + 1) * 4;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)route_f32_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(route_f32_kernel, dim3(grid), dim3(kThreads), lds, s, a);
    return hipGetLastError();
  }
  switch (cdiv(E, 16)) {
    case 1: return launch_nb<1>(a, grid, s);
    case 2: return launch_nb<2>(a, grid, s);
    case 3: return launch_nb<3>(a, grid, s);
    case 4: return launch_nb<4>(a, grid, s);
    case 5: return launch_nb<5>(a, grid, s);
    case 6: return launch_nb<6>(a, grid, s);
    case 7: return launch_nb<7>(a, grid, s);
    case 8: return launch_nb<8>(a, grid, s);
    case 9: return launch_nb<9>(a, grid, s);
    case 10: return launch_nb<10>(a, grid, s);
    case 11: return launch_nb<11>(a, grid, s);
    case 12: return launch_nb<12>(a, grid, s);
    case 13: return launch_nb<13>(a, grid, s);
    case 14: return launch_nb<14>(a, grid, s);
    case 15: return launch_nb<15>(a, grid, s);
    default: return launch_nb<16>(a, grid, s);
  }
}

}  // namespace moe
