// Router: logits, softmax top-k selection and weights, one pass over x.
//
// Top-k expert choice per token: DisagMoE technical summary, "2.2 AF-Pipe".
//
// bf16 path.  The logits L = x W_r are a skinny contraction (E <= 256
// columns) bound by reading x from HBM once:
//   1. a small pre-pass writes W_r transposed (K contiguous, [E_pad, d], zero
//      rows past E) into the caller's workspace; it is at most d * 256 * 2
//      bytes and stays in L2 for the main pass;
//   2. a workgroup of 4 wave64s takes 16 * MB tokens; the 4 waves split K
//      four ways, and each wave streams its token rows (A operand, 16
//      contiguous K-bytes per lane) and the transposed W_r rows (B operand,
//      likewise) straight from memory into v_mfma_f32_16x16x32_bf16 -- no LDS
//      staging, no barrier in the loop.  bf16 products are exact in fp32;
//      sums are fp32;
//   3. the four partial logits are added in wave order (deterministic), the
//      bias added, and the result kept in LDS for the selection.
//
// Selection and weights: 4 lanes serve one token and each scans every 4th
// expert.  The j-th pick is the best (value desc, index asc) among experts
// strictly below the (j-1)-th pick in that order, so no pick is ever marked;
// exactly equal logits go to the lower index.
#include "moe_internal.h"

namespace moe {
namespace {

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

// Softmax top-k over `ntok` logits rows in LDS: 16 lanes per token, each
// holding NV = Ep / 16 of the row's logits in registers (expert q + 16 u for
// lane q; padded experts hold -inf).  Waves take groups of 4 tokens in turn.
// The j-th pick is the best (value desc, index asc) strictly below the
// (j-1)-th pick in that order, found by a per-lane scan and a 16-lane
// reduction, so no pick is ever marked and exactly equal logits go to the
// lower index.  With renormalisation the unnormalised weights are written
// first and divided by their sum afterwards (by the same lane).
template <int NV>
__device__ __forceinline__ void select_and_weigh(const float* ll, int lstride, const RouteArgs& a,
                                                 int t_base, int ntok) {
  const int lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int q = lane & 15;
  const int E = a.E, k = a.k;
  for (int g0 = (threadIdx.x >> 6) * 4; g0 < ntok; g0 += nwaves * 4) {
    const int tt = g0 + (lane >> 4);
    const int t = t_base + tt;
    const bool live = tt < ntok;
    const float* row = ll + (live ? tt : 0) * lstride;
    float v[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = q + 16 * u;
      v[u] = (e < E) ? row[e] : -INFINITY;
    }
    // softmax denominator relative to the row max
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < NV; ++u) m = fmaxf(m, v[u]);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < NV; ++u) sum += (q + 16 * u < E) ? __expf(v[u] - m) : 0.f;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off);

    float pv = INFINITY, sel = 0.f;
    int pe = -1;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int e = q + 16 * u;
        const bool below = (v[u] < pv) || (v[u] == pv && e > pe);
        const bool better = (v[u] > bv) || (v[u] == bv && e < be);
        if (e < E && below && better) {
          bv = v[u];
          be = e;
        }
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
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
      sel += ex;
      if (q == 0 && live && t < a.T) {
        a.idx[(size_t)t * k + j] = be;
        a.w[(size_t)t * k + j] = a.renorm ? ex : ex / sum;
      }
    }
    if (a.renorm && q == 0 && live && t < a.T) {
      for (int j = 0; j < k; ++j) a.w[(size_t)t * k + j] = a.w[(size_t)t * k + j] / sel;
    }
  }
}

__device__ __forceinline__ void write_logits(const float* ll, int lstride, const RouteArgs& a,
                                             int t_base, int ntok) {
  if (a.logits_out == nullptr) return;
  const int n = ntok * a.E;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int tt = i / a.E, e = i - tt * a.E;
    const int t = t_base + tt;
    if (t < a.T) a.logits_out[(size_t)t * a.E + e] = ll[tt * lstride + e];
  }
}

// W_t[e, k] = W_r[k, e] for e < E, 0 for E <= e < Ep (d % 8 == 0).  Thread
// (kc, e) gathers rows 8 kc .. 8 kc + 7 of column e and writes them as one
// 16-byte vector; consecutive threads take consecutive experts, so each row
// read of a wave is contiguous.
__global__ __launch_bounds__(kThreads) void transpose_router_kernel(const bf16_t* __restrict__ W,
                                                                   int d, int E, int Ep,
                                                                   bf16_t* __restrict__ Wt) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= (d / 8) * Ep) return;
  const int e = i % Ep, kc = i / Ep;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (e < E) {
    const bf16_t* src = W + (size_t)kc * 8 * E + e;
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r >> 1] |= (uint32_t)src[(size_t)r * E] << (16 * (r & 1));
  }
  *reinterpret_cast<u32x4*>(Wt + (size_t)e * d + (size_t)kc * 8) = v;
}

// NB = ceil(E / 16) column blocks of 16 experts; MB = token blocks of 16 per
// workgroup; NWV waves split K (more waves = more loads in flight per CU: the
// kernel is bound by streaming x once from HBM).
template <int NB, int MB, int NWV>
__global__ __launch_bounds__(NWV * 64) void route_bf16_kernel(RouteArgs a, const bf16_t* __restrict__ Wt) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int Ep = NB * 16;
  constexpr int TW = MB * 16;   // tokens per workgroup
  constexpr int ls = Ep + 1;    // LDS row stride of the logits, in floats
  constexpr int NT = NWV * 64;
  float* part = reinterpret_cast<float*>(smem);  // [NWV][TW][Ep] partial logits
  float* ll = part;                               // [TW][ls] logits (reuses part)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: K bounds in SGPRs
  const int t_base = blockIdx.x * TW;
  const int d = a.d, E = a.E;
  const int kq = cdiv(cdiv(d, NWV), 32) * 32;  // K per wave, a multiple of 32
  const int kb = wave * kq, ke = min(d, kb + kq);

  const bf16_t* xr[MB];
  bool t_ok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = t_base + mb * 16 + (lane & 15);
    t_ok[mb] = t < a.T;
    xr[mb] = static_cast<const bf16_t*>(a.x) + (size_t)(t_ok[mb] ? t : 0) * d;
  }
  const bf16_t* wr[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wr[nb] = Wt + (size_t)(nb * 16 + (lane & 15)) * d;

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K in chunks of ST steps of 32: all loads of a chunk are issued before its
  // MFMAs, so each wave keeps ST (MB + NB) 1 KiB loads in flight
  constexpr int ST = (MB + NB) <= 2 ? 8 : (MB + NB) <= 8 ? 4 : 2;
  const bf16x8 zero8 = {};
  // rows of tokens past T read token 0 (xr); their logits are never stored
  for (int k0 = kb; k0 < ke; k0 += 32 * ST) {
    bf16x8 av[ST][MB], bv[ST][NB];
    if (k0 + 32 * ST <= ke) {
      // the whole chunk lies inside K: no predicates
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        const int kk = k0 + st * 32 + (lane >> 4) * 8;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) av[st][mb] = *reinterpret_cast<const bf16x8*>(xr[mb] + kk);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bv[st][nb] = *reinterpret_cast<const bf16x8*>(wr[nb] + kk);
      }
    } else {
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        const int kk = k0 + st * 32 + (lane >> 4) * 8;
        const bool kin = kk < ke;  // d % 8 == 0: a lane's 8 values are all in or all out
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          av[st][mb] = kin ? *reinterpret_cast<const bf16x8*>(xr[mb] + kk) : zero8;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          bv[st][nb] = kin ? *reinterpret_cast<const bf16x8*>(wr[nb] + kk) : zero8;
      }
    }
#pragma unroll
    for (int st = 0; st < ST; ++st)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[st][mb], bv[st][nb], acc[mb][nb], 0, 0, 0);
  }

  // accumulator lane layout of a 16x16 block: column lane % 16, rows
  // 4 * (lane / 16) + i
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = mb * 16 + (lane >> 4) * 4 + i;
        part[(wave * TW + tt) * Ep + nb * 16 + (lane & 15)] = acc[mb][nb][i];
      }
  __syncthreads();
  // sum the K parts in wave order, add the bias
  constexpr int PER = (TW * Ep + NT - 1) / NT;
  float lv[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * NT;
    float v = 0.f;
    if (i < TW * Ep) {
      const int e = i % Ep;
#pragma unroll
      for (int w = 0; w < NWV; ++w) v += part[w * TW * Ep + i];
      if (a.bias && e < E) v += a.bias[e];
    }
    lv[u] = v;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * NT;
    if (i < TW * Ep) ll[(i / Ep) * ls + (i % Ep)] = lv[u];
  }
  __syncthreads();
  write_logits(ll, ls, a, t_base, TW);
  select_and_weigh<NB>(ll, ls, a, t_base, TW);
}

// fp32 path (small layers): plain sequential FMA dot products, 64 tokens
// per workgroup.
template <int NV>
__global__ __launch_bounds__(kThreads) void route_f32_kernel(RouteArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int kTok = 64;
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
  write_logits(ll, ls, a, t_base, kTok);
  select_and_weigh<NV>(ll, ls, a, t_base, kTok);
}

template <int NB, int MB, int NWV>
hipError_t launch_nb_mb(const RouteArgs& a, const bf16_t* Wt, hipStream_t s) {
  constexpr int Ep = NB * 16, TW = MB * 16;
  const size_t lds = (size_t)NWV * TW * Ep * 4;  // >= TW * (Ep + 1) * 4, the logits reuse it
  static_assert((size_t)NWV * TW * Ep * 4 <= 65536, "partial logits fit 64 KiB");
  hipLaunchKernelGGL((route_bf16_kernel<NB, MB, NWV>), dim3(cdiv(a.T, TW)), dim3(NWV * 64), lds, s,
                     a, Wt);
  return hipGetLastError();
}

// Token blocks per workgroup (MB) and K-splitting waves (NWV): the kernel
// streams x once, so it wants many loads in flight -- about 16 waves per
// CU -- while the partial logits [NWV][16 MB][Ep] stay within 64 KiB and
// each workgroup reads the transposed W_r (from L2) once per 16 MB tokens.
template <int NB>
hipError_t launch_nb(const RouteArgs& a, const bf16_t* Wt, hipStream_t s) {
  constexpr int Ep = NB * 16;
  constexpr int NW16 = (16 * 16 * Ep * 4 <= 65536) ? 16 : (8 * 16 * Ep * 4 <= 65536) ? 8 : 4;
  constexpr int NW32 = (16 * 32 * Ep * 4 <= 65536) ? 16 : (8 * 32 * Ep * 4 <= 65536) ? 8 : 4;
  if constexpr (4 * 64 * Ep * 4 <= 65536) {
    // 4 token blocks for long batches: a quarter of the W_r reads per token
    if (a.T >= 256 * 64) return launch_nb_mb<NB, 4, 4>(a, Wt, s);
  }
  if constexpr (4 * 32 * Ep * 4 <= 65536) {
    if (a.T >= 256 * 32) {
      // 2 token blocks: fewer reads of W_r per token
      if (a.T >= 256 * 32 * 4) return launch_nb_mb<NB, 2, (NW32 > 4 ? 4 : NW32)>(a, Wt, s);
      return launch_nb_mb<NB, 2, (NW32 > 8 ? 8 : NW32)>(a, Wt, s);
    }
  }
  if (a.T >= 256 * 16 * 2) return launch_nb_mb<NB, 1, (NW16 > 8 ? 8 : NW16)>(a, Wt, s);
  return launch_nb_mb<NB, 1, NW16>(a, Wt, s);
}

}  // namespace

size_t route_workspace_bytes(int d, int E, bool bf16) {
  if (!bf16) return 0;
  return align_up((size_t)cdiv(E, 16) * 16 * d * sizeof(bf16_t), 256);
}

hipError_t launch_route(const void* x, const void* W_r, const float* bias, int T, int d, int E,
                        int k, bool renorm, bool bf16, int32_t* idx, float* w, float* logits_out,
                        void* ws, hipStream_t s) {
  RouteArgs a{x, W_r, bias, T, d, E, k, renorm ? 1 : 0, idx, w, logits_out};
  if (!bf16) {
    const size_t lds = (size_t)64 * (E + 1) * 4;  // <= 64 * 257 * 4 = 65792 bytes
    auto launch = [&](auto kern) -> hipError_t {
      if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(kern, dim3(cdiv(T, 64)), dim3(kThreads), lds, s, a);
      return hipGetLastError();
    };
    // logits per lane in the selection: E / 16 rounded up
    if (E <= 16) return launch(route_f32_kernel<1>);
    if (E <= 32) return launch(route_f32_kernel<2>);
    if (E <= 64) return launch(route_f32_kernel<4>);
    return launch(route_f32_kernel<16>);
  }
  const int Ep = cdiv(E, 16) * 16;
  bf16_t* Wt = static_cast<bf16_t*>(ws);
  hipLaunchKernelGGL(transpose_router_kernel, dim3(cdiv((d / 8) * Ep, kThreads)), dim3(kThreads),
                     0, s, static_cast<const bf16_t*>(W_r), d, E, Ep, Wt);
  switch (Ep / 16) {
    case 1: return launch_nb<1>(a, Wt, s);
    case 2: return launch_nb<2>(a, Wt, s);
    case 3: return launch_nb<3>(a, Wt, s);
    case 4: return launch_nb<4>(a, Wt, s);
    case 5: return launch_nb<5>(a, Wt, s);
    case 6: return launch_nb<6>(a, Wt, s);
    case 7: return launch_nb<7>(a, Wt, s);
    case 8: return launch_nb<8>(a, Wt, s);
    case 9: return launch_nb<9>(a, Wt, s);
    case 10: return launch_nb<10>(a, Wt, s);
    case 11: return launch_nb<11>(a, Wt, s);
    case 12: return launch_nb<12>(a, Wt, s);
    case 13: return launch_nb<13>(a, Wt, s);
    case 14: return launch_nb<14>(a, Wt, s);
    case 15: return launch_nb<15>(a, Wt, s);
    default: return launch_nb<16>(a, Wt, s);
  }
}

}  // namespace moe
