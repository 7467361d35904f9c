// Memory-bound backward kernels of the MoE layer: combine, unpermute, top-k
// weights and the router's (or shared gate's) skinny linear map.
//
// The layer is trained (COMET page, "What Is COMET"; DisagMoE page, "2.2
// AF-Pipe", backward stream); these are the gradients of its combine
// (DisagMoE page, "2.2 AF-Pipe": top-k weighted combine), of the dispatch
// (unpermute: each token sums the gradients of its k permuted rows) and of
// the top-k router:
//   combine:  dw[t,j] = <dy[t], y_perm[inv[t,j]]>,  dy_perm[inv[t,j]] = w[t,j] dy[t];
//             shared term g S: dy_shared = g dy, dgate[t] = <dy[t], S[t]> g (1 - g);
//   weights:  renormalised: dL[e_j] = w_j (dw_j - sum_i w_i dw_i), 0 elsewhere;
//             otherwise:    dL[e] = p_e ([e = e_j] dw_j - sum_i p_{e_i} dw_i);
//   linear:   dW = x^T G, db = sum_t G[t], dx += G W^T  (G = dL, or the gate's dz).
// Every sum runs in a fixed order (block reductions in wave order, partial
// sums over token chunks added in chunk order): results are deterministic.
#include "moe_internal.h"

#include <algorithm>

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// 4 scaled values to the row-major output (bf16 RNE or fp32), vector index c
template <typename OT>
__device__ __forceinline__ void store4(OT* out, size_t c, const f32x4 s) {
  if (sizeof(OT) == 2) {
    uint2 o;
    o.x = pack_bf16x2(s[0], s[1]);
    o.y = pack_bf16x2(s[2], s[3]);
    *reinterpret_cast<uint2*>(out + c * 4) = o;
  } else {
    *reinterpret_cast<f32x4*>(out + c * 4) = s;
  }
}

// one workgroup per token; KS = k (1..8); OT: storage type of dy_perm, dy_shared
template <int KS, typename OT>
__global__ __launch_bounds__(kThreads) void combine_backward_kernel(
    const f32x4* __restrict__ dy, const f32x4* __restrict__ y_perm, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, int vecs, const f32x4* __restrict__ y_shared,
    const float* __restrict__ gate_logit, OT* __restrict__ dy_perm, float* __restrict__ dw,
    OT* __restrict__ dy_shared, float* __restrict__ dgate) {
  __shared__ float red[kThreads / 64][KS + 1];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int r[KS];
  float w[KS], dot[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    r[j] = inv[(size_t)t * KS + j];
    w[j] = topk_w[(size_t)t * KS + j];
    dot[j] = 0.f;
  }
  float g = 1.f, dot_s = 0.f;
  if (gate_logit) g = 1.f / (1.f + __expf(-gate_logit[t]));
  for (int c = threadIdx.x; c < vecs; c += kThreads) {
    const f32x4 v = dy[(size_t)t * vecs + c];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const f32x4 yp = y_perm[(size_t)r[j] * vecs + c];
      dot[j] += v[0] * yp[0] + v[1] * yp[1] + v[2] * yp[2] + v[3] * yp[3];
      store4(dy_perm, (size_t)r[j] * vecs + c, w[j] * v);
    }
    if (dy_shared) {
      store4(dy_shared, (size_t)t * vecs + c, g * v);
      if (dgate) {
        const f32x4 ys = y_shared[(size_t)t * vecs + c];
        dot_s += v[0] * ys[0] + v[1] * ys[1] + v[2] * ys[2] + v[3] * ys[3];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const float s = wave_sum(dot[j]);
    if (lane == 0) red[wave][j] = s;
  }
  {
    const float s = wave_sum(dot_s);
    if (lane == 0) red[wave][KS] = s;
  }
  __syncthreads();
  if (threadIdx.x <= KS) {
    const int j = threadIdx.x;
    float s = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kThreads / 64; ++w2) s += red[w2][j];
    if (j < KS) dw[(size_t)t * KS + j] = s;
    else if (dgate) dgate[t] = s * g * (1.f - g);
  }
}

// Any k (the forward takes up to 256 slots): the slots one after another,
// each slot's dot product reduced over the workgroup before the next; the
// same per-thread, per-wave and cross-wave order as the kernel above.
template <typename OT>
__global__ __launch_bounds__(kThreads) void combine_backward_any_kernel(
    const f32x4* __restrict__ dy, const f32x4* __restrict__ y_perm, const int32_t* __restrict__ inv,
    const float* __restrict__ topk_w, int vecs, int k, const f32x4* __restrict__ y_shared,
    const float* __restrict__ gate_logit, OT* __restrict__ dy_perm, float* __restrict__ dw,
    OT* __restrict__ dy_shared, float* __restrict__ dgate) {
  __shared__ float red[kThreads / 64];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float g = 1.f;
  if (gate_logit) g = 1.f / (1.f + __expf(-gate_logit[t]));
  for (int j = 0; j < k; ++j) {
    const int r = inv[(size_t)t * k + j];
    const float w = topk_w[(size_t)t * k + j];
    float dot = 0.f;
    for (int c = threadIdx.x; c < vecs; c += kThreads) {
      const f32x4 v = dy[(size_t)t * vecs + c];
      const f32x4 yp = y_perm[(size_t)r * vecs + c];
      dot += v[0] * yp[0] + v[1] * yp[1] + v[2] * yp[2] + v[3] * yp[3];
      store4(dy_perm, (size_t)r * vecs + c, w * v);
    }
    const float sw = wave_sum(dot);
    if (lane == 0) red[wave] = sw;
    __syncthreads();
    if (threadIdx.x == 0) {
      float tot = 0.f;
      for (int w2 = 0; w2 < kThreads / 64; ++w2) tot += red[w2];
      dw[(size_t)t * k + j] = tot;
    }
    __syncthreads();  // red is reused by the next slot
  }
  if (dy_shared) {
    float dot_s = 0.f;
    for (int c = threadIdx.x; c < vecs; c += kThreads) {
      const f32x4 v = dy[(size_t)t * vecs + c];
      store4(dy_shared, (size_t)t * vecs + c, g * v);
      if (dgate) {
        const f32x4 ys = y_shared[(size_t)t * vecs + c];
        dot_s += v[0] * ys[0] + v[1] * ys[1] + v[2] * ys[2] + v[3] * ys[3];
      }
    }
    if (dgate) {
      const float sw = wave_sum(dot_s);
      if (lane == 0) red[wave] = sw;
      __syncthreads();
      if (threadIdx.x == 0) {
        float tot = 0.f;
        for (int w2 = 0; w2 < kThreads / 64; ++w2) tot += red[w2];
        dgate[t] = tot * g * (1.f - g);
      }
    }
  }
}

// The combine backward over compact rows (layer 1's fp16 output with one
// power-of-two factor per 32-column segment): the same gradients. The factor
// is a power of two, so <dy, h * f> = f <dy, h> exactly (no overflow at these
// magnitudes): each 8-column dot is taken on the fp16 values and scaled once.
// 8 columns per step: two 16-byte vectors of dy, one of a row.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float dot8(const f32x4 a, const f32x4 b, const u32x4 raw, float fac) {
  const f16x8 h = __builtin_bit_cast(f16x8, raw);
  float s = a[0] * static_cast<float>(h[0]) + a[1] * static_cast<float>(h[1]) +
            a[2] * static_cast<float>(h[2]) + a[3] * static_cast<float>(h[3]);
  s += b[0] * static_cast<float>(h[4]) + b[1] * static_cast<float>(h[5]) +
       b[2] * static_cast<float>(h[6]) + b[3] * static_cast<float>(h[7]);
  return s * fac;
}

// one workgroup per token; KS = k (1..8): one pass over dy for every slot and
// the shared term; KS = 0: any k, the slots one after another (each slot's
// dot reduced over the workgroup before the next), then the shared term
template <int KS, typename OT>
__global__ __launch_bounds__(kThreads) void combine_backward_f16_kernel(
    const f32x4* __restrict__ dy, const u32x4* __restrict__ y_h, const float* __restrict__ y_s,
    const int32_t* __restrict__ inv, const float* __restrict__ topk_w, int chunks, int k,
    const u32x4* __restrict__ ys_h, const float* __restrict__ ys_s,
    const float* __restrict__ gate_logit, OT* __restrict__ dy_perm, float* __restrict__ dw,
    OT* __restrict__ dy_shared, float* __restrict__ dgate) {
  constexpr bool kOne = KS > 0;     // every slot in one pass
  constexpr int NS = kOne ? KS : 1;  // slots per pass
  __shared__ float red[kThreads / 64][NS + 1];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int segs = chunks >> 2;
  const int kk = kOne ? KS : k;
  const f32x4* dyt = dy + (size_t)t * chunks * 2;
  float g = 1.f;
  if (gate_logit) g = 1.f / (1.f + __expf(-gate_logit[t]));
  float dot_s = 0.f;
  for (int j0 = 0; j0 < kk; j0 += NS) {
    int r[NS];
    float w[NS], dot[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      r[j] = inv[(size_t)t * kk + j0 + j];
      w[j] = topk_w[(size_t)t * kk + j0 + j];
      dot[j] = 0.f;
    }
    for (int c = threadIdx.x; c < chunks; c += kThreads) {
      const f32x4 v0 = dyt[2 * c], v1 = dyt[2 * c + 1];
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        dot[j] += dot8(v0, v1, y_h[(size_t)r[j] * chunks + c], y_s[(size_t)r[j] * segs + (c >> 2)]);
        store4(dy_perm, (size_t)r[j] * chunks * 2 + 2 * c, w[j] * v0);
        store4(dy_perm, (size_t)r[j] * chunks * 2 + 2 * c + 1, w[j] * v1);
      }
      if (kOne && dy_shared) {
        store4(dy_shared, (size_t)t * chunks * 2 + 2 * c, g * v0);
        store4(dy_shared, (size_t)t * chunks * 2 + 2 * c + 1, g * v1);
        if (dgate)
          dot_s += dot8(v0, v1, ys_h[(size_t)t * chunks + c], ys_s[(size_t)t * segs + (c >> 2)]);
      }
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float sw = wave_sum(dot[j]);
      if (lane == 0) red[wave][j] = sw;
    }
    __syncthreads();
    if (threadIdx.x < NS) {
      float s = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kThreads / 64; ++w2) s += red[w2][threadIdx.x];
      dw[(size_t)t * kk + j0 + threadIdx.x] = s;
    }
    __syncthreads();  // red is reused below
  }
  if (!kOne && dy_shared) {
    for (int c = threadIdx.x; c < chunks; c += kThreads) {
      const f32x4 v0 = dyt[2 * c], v1 = dyt[2 * c + 1];
      store4(dy_shared, (size_t)t * chunks * 2 + 2 * c, g * v0);
      store4(dy_shared, (size_t)t * chunks * 2 + 2 * c + 1, g * v1);
      if (dgate)
        dot_s += dot8(v0, v1, ys_h[(size_t)t * chunks + c], ys_s[(size_t)t * segs + (c >> 2)]);
    }
  }
  if (dgate) {
    const float sw = wave_sum(dot_s);
    if (lane == 0) red[wave][0] = sw;
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kThreads / 64; ++w2) s += red[w2][0];
      dgate[t] = s * g * (1.f - g);
    }
  }
}

// dx[t] (+)= sum_j dx_perm[inv[t, j]] (slot order); one workgroup per token
template <int KS>
__global__ __launch_bounds__(kThreads) void unpermute_kernel(const f32x4* __restrict__ dx_perm,
                                                             const int32_t* __restrict__ inv,
                                                             int vecs, int accumulate,
                                                             f32x4* __restrict__ dx) {
  const int t = blockIdx.x;
  int r[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) r[j] = inv[(size_t)t * KS + j];
  for (int c = threadIdx.x; c < vecs; c += kThreads) {
    f32x4 v = accumulate ? dx[(size_t)t * vecs + c] : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j) s += dx_perm[(size_t)r[j] * vecs + c];
    dx[(size_t)t * vecs + c] = v + s;
  }
}

// any k: the same sum with the slot loop at run time
__global__ __launch_bounds__(kThreads) void unpermute_any_kernel(const f32x4* __restrict__ dx_perm,
                                                                 const int32_t* __restrict__ inv,
                                                                 int vecs, int k, int accumulate,
                                                                 f32x4* __restrict__ dx) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < vecs; c += kThreads) {
    f32x4 v = accumulate ? dx[(size_t)t * vecs + c] : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) s += dx_perm[(size_t)inv[(size_t)t * k + j] * vecs + c];
    dx[(size_t)t * vecs + c] = v + s;
  }
}

// dL [T, E] from the fp32 logits, the selection and dw.  LPT lanes per token
// (a power of two >= E, at most 64): lane li takes experts li, li + LPT, ...
// (at most 4, E <= 256), so a token's logits are read and dL written
// contiguously; its max and sums are xor-shuffle reductions over its lanes
// (a fixed order).  Renormalised: w_j = softmax over the k selected logits,
// dL[e_j] = w_j (dw_j - s), s = sum_j w_j dw_j, 0 elsewhere; otherwise
// p = softmax over all E, dL[e] = p_e ([e = e_j] dw_j - s), s = sum_j p_{e_j} dw_j.
template <int LPT>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = LPT / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = LPT / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
template <int LPT>
__global__ __launch_bounds__(kThreads) void topk_weights_backward_kernel(
    const float* __restrict__ L, const int32_t* __restrict__ idx, const float* __restrict__ dw,
    int T, int E, int k, int renorm, float* __restrict__ dL) {
  constexpr int NE = 4;
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  const int t = gid / LPT, li = gid % LPT;
  const bool live = t < T;
  const int tt = live ? t : 0;  // every lane takes part in the shuffles
  const float* Lt = L + (size_t)tt * E;
  float lv[NE], dsel[NE];
  bool sel[NE], in[NE];
#pragma unroll
  for (int r = 0; r < NE; ++r) {
    const int e = li + LPT * r;
    in[r] = e < E;
    lv[r] = in[r] ? Lt[e] : 0.f;
    sel[r] = false;
    dsel[r] = 0.f;
  }
  for (int j = 0; j < k; ++j) {
    const int ej = idx[(size_t)tt * k + j];
    const float dj = dw[(size_t)tt * k + j];
#pragma unroll
    for (int r = 0; r < NE; ++r)
      if (li + LPT * r == ej) {
        sel[r] = true;
        dsel[r] = dj;
      }
  }
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < NE; ++r)
    if (in[r] && (!renorm || sel[r])) m = fmaxf(m, lv[r]);
  m = group_max<LPT>(m);
  float q[NE], z = 0.f;
#pragma unroll
  for (int r = 0; r < NE; ++r) {
    q[r] = in[r] && (!renorm || sel[r]) ? __expf(lv[r] - m) : 0.f;
    z += q[r];
  }
  z = group_sum<LPT>(z);
  float sp = 0.f;
#pragma unroll
  for (int r = 0; r < NE; ++r)
    if (sel[r]) sp += q[r] / z * dsel[r];
  sp = group_sum<LPT>(sp);
  if (!live) return;
  float* out = dL + (size_t)t * E;
#pragma unroll
  for (int r = 0; r < NE; ++r)
    if (in[r]) {
      const float pe = q[r] / z;
      out[li + LPT * r] = renorm ? (sel[r] ? pe * (dsel[r] - sp) : 0.f) : pe * (dsel[r] - sp);
    }
}

// dW partials (register-blocked fp32): a block takes EB experts, XCB
// columns (512, or 256 for EB = 64) and token chunk tc of tc_len tokens.
// Thread (token slice ts, expert group eg, column group cg) accumulates an
// 8 x 8 block over the rows ts, ts + TS, ... of each staged group of rows,
//   acc[c][j] += x[t, c0 + 8 cg + c] G[t, e0 + 8 eg + j],
// and the TS slices are then added in slice order through LDS (TS = 4, 2
// for EB = 8, 16: the same partial sums with more threads in flight), and
// written to part[tc][column][expert].  x row segments (16 bytes, coalesced
// over the column groups) come from global memory, 8 rows in flight; G rows
// are staged in LDS 32 at a time and read as broadcasts.  EB: the smallest
// of 8, 16, 32, 64 covering E (E > 64 loops over 64-expert chunks).
constexpr int GR = 32;  // G rows per LDS stage
template <int EB>
struct XtgShape {
  static constexpr int EG = EB / 8;                   // expert groups
  static constexpr int TS = EB == 8 ? 4 : EB == 16 ? 2 : 1;  // token slices
  static constexpr int CG = kThreads / (EG * TS);     // column groups
  static constexpr int CB = 8 * CG;                   // columns per block
};
template <typename XT, int EB>
__global__ __launch_bounds__(kThreads) void xtg_partial_kernel(const XT* __restrict__ x,
                                                               const float* __restrict__ G, int T,
                                                               int d, int E, int tc_len,
                                                               float* __restrict__ part) {
  using S = XtgShape<EB>;
  constexpr int EG = S::EG, TS = S::TS, CG = S::CG, CB = S::CB;
  __shared__ __attribute__((aligned(16))) float gs[GR][EB];
  __shared__ __attribute__((aligned(16))) float red[TS > 1 ? (TS - 1) * CG * EG * 64 : 1];
  const int cg = threadIdx.x % CG, eg = (threadIdx.x / CG) % EG, ts = threadIdx.x / (CG * EG);
  const int col = blockIdx.x * CB + 8 * cg;
  const bool col_ok = col < d;  // d is a multiple of 8: a column group is whole or absent
  const int tc = blockIdx.y;
  const int t0 = tc * tc_len, t1 = min(T, t0 + tc_len);
  for (int e0 = 0; e0 < E; e0 += EB) {
    const int ne = min(EB, E - e0);
    float acc[8][8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[c][j] = 0.f;
    for (int tb = t0; tb < t1; tb += GR) {
      const int nt = min(GR, t1 - tb);
      __syncthreads();
      for (int q = threadIdx.x; q < GR * EB; q += kThreads) {
        const int rr = q / EB, e = q % EB;
        gs[rr][e] = (rr < nt && e < ne) ? G[(size_t)(tb + rr) * E + e0 + e] : 0.f;
      }
      __syncthreads();
      if (col_ok) {
        // this slice's rows ts, ts + TS, ...: 8 of them loaded before their
        // arithmetic (rows past the stage read row tb, and are not used)
        for (int rb = ts; rb < nt; rb += 8 * TS) {
          u32x4 xr[8][sizeof(XT) == 2 ? 1 : 2];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int rr = rb + u * TS < nt ? rb + u * TS : 0;
            const XT* xp = x + (size_t)(tb + rr) * d + col;
            xr[u][0] = *reinterpret_cast<const u32x4*>(xp);
            if (sizeof(XT) == 4) xr[u][sizeof(XT) == 2 ? 0 : 1] = *reinterpret_cast<const u32x4*>(xp + 4);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int rr = rb + u * TS;
            if (rr >= nt) break;
            float xv[8];
            if (sizeof(XT) == 2) {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                xv[2 * c] = __uint_as_float(xr[u][0][c] << 16);
                xv[2 * c + 1] = __uint_as_float(xr[u][0][c] & 0xffff0000u);
              }
            } else {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                xv[c] = __uint_as_float(xr[u][0][c]);
                xv[4 + c] = __uint_as_float(xr[u][sizeof(XT) == 2 ? 0 : 1][c]);
              }
            }
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(&gs[rr][8 * eg]);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(&gs[rr][8 * eg + 4]);
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
              for (int j = 0; j < 8; ++j)
                acc[c][j] = fmaf(xv[c], j < 4 ? g0[j] : g1[j - 4], acc[c][j]);
          }
        }
      }
    }
    if (TS > 1) {
      // slices 1 .. TS - 1 hand their sums to slice 0, which adds them in order
      const int slot = threadIdx.x % (CG * EG);
      __syncthreads();
      if (ts > 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int j = 0; j < 8; ++j) red[((ts - 1) * CG * EG + slot) * 64 + c * 8 + j] = acc[c][j];
      }
      __syncthreads();
      if (ts == 0) {
        for (int s2 = 1; s2 < TS; ++s2)
#pragma unroll
          for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[c][j] += red[((s2 - 1) * CG * EG + slot) * 64 + c * 8 + j];
      }
    }
    if (col_ok && ts == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (8 * eg + j < ne) part[((size_t)tc * d + col + c) * E + e0 + 8 * eg + j] = acc[c][j];
    }
  }
}

// expert block of the dW partials for E experts, and its columns per block
int xtg_eb(int E) { return E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64; }
int xtg_cols(int E) {
  const int eb = xtg_eb(E);
  return eb == 8 ? XtgShape<8>::CB : eb == 16 ? XtgShape<16>::CB : eb == 32 ? XtgShape<32>::CB
                                                                           : XtgShape<64>::CB;
}

// tokens per partial chunk: about 1024 blocks over (column blocks x token
// chunks), a multiple of GR between GR and 512
int xtg_chunk(int T, int d, int E) {
  const long long want = (long long)T * cdiv(d, xtg_cols(E)) / 1024;
  return (int)std::min<long long>(512, std::max<long long>(GR, (want + GR - 1) / GR * GR));
}

// dW[i, e] = sum over chunks (in order) of part[c][i][e]
__global__ __launch_bounds__(kThreads) void sum_chunks_kernel(const float* __restrict__ part,
                                                              int nc, size_t n,
                                                              float* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  int c = 0;
  for (; c + 8 <= nc; c += 8) {  // 8 loads in flight, added in chunk order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(c + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; c < nc; ++c) s += part[(size_t)c * n + i];
  out[i] = s;
}

// db[e] = sum_t G[t, e] (one workgroup per expert, wave-order reduction)
__global__ __launch_bounds__(kThreads) void colsum_kernel(const float* __restrict__ G, int T,
                                                          int E, float* __restrict__ db) {
  __shared__ float red[kThreads / 64];
  const int e = blockIdx.x;
  float s = 0.f;
  for (int t = threadIdx.x; t < T; t += kThreads) s += G[(size_t)t * E + e];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = 0.f;
    for (int w2 = 0; w2 < kThreads / 64; ++w2) v += red[w2];
    db[e] = v;
  }
}

// dx[t, i] += sum_e G[t, e] W[i, e] (register-blocked fp32): a block takes
// 64 tokens x 256 columns; thread (token group ty, column group tx) keeps an
// 8 x 8 block, summing over the experts in order.  Per chunk of EB experts
// (EB as for the dW partials), G is staged transposed (gs[e][t]) and W as
// its rows' chunk, transposed (ws[e][i]); a thread reads 8 tokens and 8
// columns per expert as 16-byte LDS reads (the token reads are broadcasts
// across the wave, the column reads 512 contiguous bytes).  Staging loads
// are 16 bytes wide where E and the pointers allow (rows then start
// 16-byte aligned).
constexpr int DXT = 64, DXC = 256;
template <typename WT, int EB>
__global__ __launch_bounds__(kThreads) void dx_linear_kernel(const float* __restrict__ G,
                                                             const WT* __restrict__ W, int T,
                                                             int d, int E,
                                                             float* __restrict__ dx) {
  constexpr int WV = 16 / sizeof(WT);  // W elements per 16-byte load
  __shared__ __attribute__((aligned(16))) float gs[EB][DXT + 4];
  __shared__ __attribute__((aligned(16))) WT ws[EB][DXC + 8];
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
  const int t0 = blockIdx.y * DXT, c0 = blockIdx.x * DXC;
  const bool gvec = (E % 4) == 0 && ((uintptr_t)G & 15) == 0;
  const bool wvec = (E % WV) == 0 && ((uintptr_t)W & 15) == 0;
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = 0.f;
  for (int e0 = 0; e0 < E; e0 += EB) {
    const int ne = min(EB, E - e0);
    __syncthreads();
    if (gvec) {
      for (int q = threadIdx.x; q < DXT * (EB / 4); q += kThreads) {
        const int rr = q / (EB / 4), e = (q % (EB / 4)) * 4;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (t0 + rr < T && e < ne) v = *reinterpret_cast<const f32x4*>(G + (size_t)(t0 + rr) * E + e0 + e);
#pragma unroll
        for (int j = 0; j < 4; ++j) gs[e + j][rr] = v[j];
      }
    } else {
      for (int q = threadIdx.x; q < DXT * EB; q += kThreads) {
        const int rr = q / EB, e = q % EB;
        gs[e][rr] = (t0 + rr < T && e < ne) ? G[(size_t)(t0 + rr) * E + e0 + e] : 0.f;
      }
    }
    if (wvec) {
      for (int q = threadIdx.x; q < DXC * (EB / WV); q += kThreads) {
        const int i = q / (EB / WV), e = (q % (EB / WV)) * WV;
        WT v[WV];
#pragma unroll
        for (int j = 0; j < WV; ++j) v[j] = WT(0);
        if (c0 + i < d && e < ne) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(W + (size_t)(c0 + i) * E + e0 + e);
          __builtin_memcpy(v, &raw, 16);
        }
#pragma unroll
        for (int j = 0; j < WV; ++j) ws[e + j][i] = v[j];
      }
    } else {
      for (int q = threadIdx.x; q < DXC * EB; q += kThreads) {
        const int i = q / EB, e = q % EB;
        ws[e][i] = (c0 + i < d && e < ne) ? W[(size_t)(c0 + i) * E + e0 + e] : WT(0);
      }
    }
    __syncthreads();
    for (int e = 0; e < ne; ++e) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(&gs[e][8 * ty]);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(&gs[e][8 * ty + 4]);
      float wv[8];
      if (sizeof(WT) == 2) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&ws[e][8 * tx]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          wv[2 * c] = __uint_as_float(v[c] << 16);
          wv[2 * c + 1] = __uint_as_float(v[c] & 0xffff0000u);
        }
      } else {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(&ws[e][8 * tx]);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(&ws[e][8 * tx + 4]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          wv[c] = v0[c];
          wv[4 + c] = v1[c];
        }
      }
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[a][c] = fmaf(a < 4 ? g0[a] : g1[a - 4], wv[c], acc[a][c]);
    }
  }
  const int col = c0 + 8 * tx;
  if (col >= d) return;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int t = t0 + 8 * ty + a;
    if (t >= T) continue;
    f32x4* o = reinterpret_cast<f32x4*>(dx + (size_t)t * d + col);
    f32x4 v0 = o[0], v1 = o[1];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v0[c] += acc[a][c];
      v1[c] += acc[a][4 + c];
    }
    o[0] = v0;
    o[1] = v1;
  }
}

// ---- bf16 x and W: the same two products on the matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  G is fp32: it enters as
// hi + lo with hi = bf16(G), lo = bf16(G - hi).  G - hi is exact in fp32, so
// |G - hi - lo| <= 2^-18 |G|, and every product with a bf16 x or W value is
// exact in the fp32 accumulator: the result is an fp32 sum as above, in a
// different but fixed order.
//
// G is split once, into hi and lo arrays [T, EP] whose rows are padded with
// zeros to EP = E rounded up to 64.  The operand loads then carry no guards:
// a lane whose row or column lies outside an operand reads an in-bounds
// element instead (its results are never stored), and experts past E meet
// the zeros of the G side whatever the W side reads.  A guarded load (a
// branch, or a select on the loaded value) makes the compiler wait for it
// where it is guarded, one memory round trip at a time.
typedef __attribute__((address_space(3))) bf16x4 lds_b16x4;

__host__ __device__ __forceinline__ int split_ep(int E) { return (E + 63) / 64 * 64; }

__device__ __forceinline__ void split_bf16(float g, bf16_t& hi, bf16_t& lo) {
  hi = f32_to_bf16(g);
  lo = f32_to_bf16(g - bf16_to_f32(hi));
}

// gh, gl [T, EP]: the split of G, zeros past E
__global__ __launch_bounds__(kThreads) void split_g_kernel(const float* __restrict__ G, int T,
                                                           int E, int EP, bf16_t* __restrict__ gh,
                                                           bf16_t* __restrict__ gl) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (size_t)T * EP) return;
  const int t = (int)(i / EP), e = (int)(i - (size_t)t * EP);
  split_bf16(e < E ? G[(size_t)t * E + e] : 0.f, gh[i], gl[i]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// 8 consecutive K values of one column for an MFMA operand, from a K-outer
// LDS tile (row stride ld elements): the gfx950 LDS transpose read gives
// lane l (g = l / 16) column l % 16 of rows kr .. kr + 3 (kr = 8 g + l % 16
// / 4 addressed, 4 columns per lane); two reads cover rows 8 g .. 8 g + 7.
__device__ __forceinline__ bf16x8 tr_frag(const bf16_t* tile, int ld, int kr, int col) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b16x4*)(tile + kr * ld + col));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b16x4*)(tile + (kr + 4) * ld + col));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// dW partials: part[c][i][e] = sum over the tokens t of chunk c of
// x[t, i] G[t, e].  A workgroup takes 128 columns of x, NB * 16 experts
// (blockIdx.z selects the group) and one token chunk, 32 tokens a step:
// x and G (hi, lo) are staged K-outer in LDS (rows 32 bytes longer than the
// data, against bank conflicts) and both operands are read with the
// transpose read; wave w owns columns 32 w .. 32 w + 31 (2 x NB blocks).
// The next step's global loads are issued before this step's MFMAs; G rows
// past the chunk are zeroed when staged (the x side may hold anything there).
constexpr int XM_COLS = 128, XM_K = 32, XM_LD = XM_COLS + 16;
template <int NB>
__global__ __launch_bounds__(kThreads) void xtg_mfma_kernel(const bf16_t* __restrict__ x,
                                                            const bf16_t* __restrict__ Gh,
                                                            const bf16_t* __restrict__ Gl, int T,
                                                            int d, int E, int EP, int tc_len,
                                                            float* __restrict__ part) {
  constexpr int EB = 16 * NB, GL = EB + 16;
  constexpr int GCH = XM_K * (EB / 8);  // 16-byte chunks of a G tile
  __shared__ __attribute__((aligned(16))) bf16_t xs[XM_K * XM_LD];
  __shared__ __attribute__((aligned(16))) bf16_t gh[XM_K * GL];
  __shared__ __attribute__((aligned(16))) bf16_t gl[XM_K * GL];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c0 = blockIdx.x * XM_COLS, e0 = blockIdx.z * EB;
  const int t0 = blockIdx.y * tc_len, t1 = min(T, t0 + tc_len);
  const int kr = (lane >> 4) * 8 + ((lane & 15) >> 2), cq = (lane & 3) * 4;
  // this thread's staging chunks: x rows q / 16, columns 8 (q % 16), for
  // q = tid and tid + 256; G row tid / (EB / 8), experts 8 (tid % (EB / 8))
  const int gr = threadIdx.x / (EB / 8), gc = (threadIdx.x % (EB / 8)) * 8;
  const bool gload = threadIdx.x < GCH;
  u32x4 xr[2], hr = {0u, 0u, 0u, 0u}, lr = {0u, 0u, 0u, 0u};
  bool gin = false;
  auto load = [&](int tb) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = threadIdx.x + k * kThreads, r = q >> 4, cc = (q & 15) * 8;
      const bool in = tb + r < T && c0 + cc < d;
      xr[k] = *reinterpret_cast<const u32x4*>(x + (in ? (size_t)(tb + r) * d + c0 + cc : 0));
    }
    if (gload) {
      gin = tb + gr < t1;
      const size_t off = gin ? (size_t)(tb + gr) * EP + e0 + gc : 0;
      hr = *reinterpret_cast<const u32x4*>(Gh + off);
      lr = *reinterpret_cast<const u32x4*>(Gl + off);
    }
  };
  f32x4 acc[2][NB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (t0 < t1) load(t0);
  for (int tb = t0; tb < t1; tb += XM_K) {
    __syncthreads();  // the previous step's fragment reads are done
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = threadIdx.x + k * kThreads;
      *reinterpret_cast<u32x4*>(xs + (q >> 4) * XM_LD + (q & 15) * 8) = xr[k];
    }
    if (gload) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(gh + gr * GL + gc) = gin ? hr : z;
      *reinterpret_cast<u32x4*>(gl + gr * GL + gc) = gin ? lr : z;
    }
    __syncthreads();
    if (tb + XM_K < t1) load(tb + XM_K);
    bf16x8 a[2], bh[NB], bl[NB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) a[mb] = tr_frag(xs, XM_LD, kr, 32 * w + 16 * mb + cq);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bh[nb] = tr_frag(gh, GL, kr, 16 * nb + cq);
      bl[nb] = tr_frag(gl, GL, kr, 16 * nb + cq);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], bh[nb], acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], bl[nb], acc[mb][nb], 0, 0, 0);
      }
  }
  // lane l holds columns c0 + 32 w + 16 mb + 4 (l / 16) + i, expert e0 + 16 nb + l % 16
  const int e = e0 + (lane & 15);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = c0 + 32 * w + 16 * mb + 4 * (lane >> 4) + i;
        if (col < d && e + 16 * nb < E)
          part[((size_t)blockIdx.y * d + col) * E + e + 16 * nb] = acc[mb][nb][i];
      }
}

// dx[t, i] += sum_e G[t, e] W[i, e], as C^T = W G^T: A = W (rows i, K = e),
// B = G^T (K = e, columns t).  Both are K-contiguous in memory (W [d, E],
// the split G [T, EP] row-major), so each lane loads its fragments directly:
// 8 experts of one W row (kept in registers across the tokens when E <= 32
// KS) and 8 experts of one G row; no LDS.  Wave w of a workgroup owns
// columns 64 w .. 64 w + 63 of the block's 256 and walks its tokens 64 at a
// time (4 x 4 blocks of 16 x 16).  The accumulators start from dx (lane l:
// token l % 16 of a block, 4 consecutive columns), so dx is read and written
// once, 16 bytes per lane, and the sum order is fixed: experts in order, hi
// before lo.  VEC: W rows 16-byte aligned (E a multiple of 8, W aligned).
constexpr int DM_T = 128, DM_C = 256;
template <int KS, bool VEC>
__global__ __launch_bounds__(kThreads) void dx_mfma_kernel(const bf16_t* __restrict__ Gh,
                                                           const bf16_t* __restrict__ Gl,
                                                           const bf16_t* __restrict__ W, int T,
                                                           int d, int E, int EP,
                                                           float* __restrict__ dx) {
  constexpr int EK = 32 * KS;  // experts per pass
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, l15 = lane & 15;
  const int c0 = blockIdx.x * DM_C + 64 * w;  // the wave's first column
  const int tb = blockIdx.y * DM_T;
  const int npass = cdiv(E, EK);
  bf16x8 a[4][KS];
  auto load_a = [&](int e0) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int i = c0 + 16 * mb + l15, e = e0 + 32 * ks + 8 * g;
        if (VEC) {
          const size_t off = i < d && e < E ? (size_t)i * E + e : 0;
          a[mb][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(W + off));
        } else {
          bf16_t b[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) b[j] = W[i < d && e + j < E ? (size_t)i * E + e + j : 0];
          __builtin_memcpy(&a[mb][ks], b, 16);
        }
      }
  };
  if (npass == 1) load_a(0);
  for (int sb = 0; sb < DM_T / 64; ++sb) {
    const int t0 = tb + 64 * sb;
    if (t0 >= T) break;
    f32x4 acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int t = t0 + 16 * nb + l15, col = c0 + 16 * mb + 4 * g;
        const size_t off = t < T && col < d ? (size_t)t * d + col : 0;
        acc[mb][nb] = *reinterpret_cast<const f32x4*>(dx + off);
      }
    for (int ps = 0; ps < npass; ++ps) {
      const int e0 = ps * EK;
      if (npass > 1) load_a(e0);
      bf16x8 bh[4][KS], bl[4][KS];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int t = t0 + 16 * nb + l15;
          const size_t off = (size_t)(t < T ? t : 0) * EP + e0 + 32 * ks + 8 * g;
          bh[nb][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(Gh + off));
          bl[nb][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(Gl + off));
        }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb][ks], bh[nb][ks], acc[mb][nb], 0, 0, 0);
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb][ks], bl[nb][ks], acc[mb][nb], 0, 0, 0);
          }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int t = t0 + 16 * nb + l15, col = c0 + 16 * mb + 4 * g;
        if (t < T && col < d) *reinterpret_cast<f32x4*>(dx + (size_t)t * d + col) = acc[mb][nb];
      }
  }
}

template <int KS>
void launch_cb(const float* dy, const float* y_perm, const int32_t* inv, const float* topk_w,
               int T, int d, bool bf16, const float* y_shared, const float* gate_logit,
               void* dy_perm, float* dw, void* dy_shared, float* dgate, hipStream_t s) {
  const f32x4* dyv = reinterpret_cast<const f32x4*>(dy);
  const f32x4* ypv = reinterpret_cast<const f32x4*>(y_perm);
  const f32x4* ysv = reinterpret_cast<const f32x4*>(y_shared);
  if (bf16)
    hipLaunchKernelGGL((combine_backward_kernel<KS, bf16_t>), dim3(T), dim3(kThreads), 0, s, dyv,
                       ypv, inv, topk_w, d / 4, ysv, gate_logit, static_cast<bf16_t*>(dy_perm),
                       dw, static_cast<bf16_t*>(dy_shared), dgate);
  else
    hipLaunchKernelGGL((combine_backward_kernel<KS, float>), dim3(T), dim3(kThreads), 0, s, dyv,
                       ypv, inv, topk_w, d / 4, ysv, gate_logit, static_cast<float*>(dy_perm), dw,
                       static_cast<float*>(dy_shared), dgate);
}

template <int KS>
void launch_up(const float* dx_perm, const int32_t* inv, int T, int d, bool accumulate, float* dx,
               hipStream_t s) {
  hipLaunchKernelGGL((unpermute_kernel<KS>), dim3(T), dim3(kThreads), 0, s,
                     reinterpret_cast<const f32x4*>(dx_perm), inv, d / 4, accumulate ? 1 : 0,
                     reinterpret_cast<f32x4*>(dx));
}

}  // namespace

hipError_t launch_combine_backward(const float* dy, const float* y_perm, const int32_t* inv,
                                   const float* topk_w, int T, int d, int k, bool bf16,
                                   const float* y_shared, const float* gate_logit, void* dy_perm,
                                   float* dw, void* dy_shared, float* dgate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  switch (k) {
#define MOE_CB(K) case K: launch_cb<K>(dy, y_perm, inv, topk_w, T, d, bf16, y_shared, gate_logit, dy_perm, dw, dy_shared, dgate, s); break;
    MOE_CB(1) MOE_CB(2) MOE_CB(3) MOE_CB(4) MOE_CB(5) MOE_CB(6) MOE_CB(7) MOE_CB(8)
#undef MOE_CB
    default: {
      const f32x4* dyv = reinterpret_cast<const f32x4*>(dy);
      const f32x4* ypv = reinterpret_cast<const f32x4*>(y_perm);
      const f32x4* ysv = reinterpret_cast<const f32x4*>(y_shared);
      if (bf16)
        hipLaunchKernelGGL((combine_backward_any_kernel<bf16_t>), dim3(T), dim3(kThreads), 0, s,
                           dyv, ypv, inv, topk_w, d / 4, k, ysv, gate_logit,
                           static_cast<bf16_t*>(dy_perm), dw, static_cast<bf16_t*>(dy_shared),
                           dgate);
      else
        hipLaunchKernelGGL((combine_backward_any_kernel<float>), dim3(T), dim3(kThreads), 0, s,
                           dyv, ypv, inv, topk_w, d / 4, k, ysv, gate_logit,
                           static_cast<float*>(dy_perm), dw, static_cast<float*>(dy_shared), dgate);
    }
  }
  return hipGetLastError();
}

template <int KS, typename OT>
void launch_cbh(const float* dy, const uint16_t* y_h, const float* y_s, const int32_t* inv,
                const float* topk_w, int T, int d, int k, const uint16_t* ys_h, const float* ys_s,
                const float* gate_logit, void* dy_perm, float* dw, void* dy_shared, float* dgate,
                hipStream_t s) {
  hipLaunchKernelGGL((combine_backward_f16_kernel<KS, OT>), dim3(T), dim3(kThreads), 0, s,
                     reinterpret_cast<const f32x4*>(dy), reinterpret_cast<const u32x4*>(y_h), y_s,
                     inv, topk_w, d / 8, k, reinterpret_cast<const u32x4*>(ys_h), ys_s, gate_logit,
                     static_cast<OT*>(dy_perm), dw, static_cast<OT*>(dy_shared), dgate);
}

hipError_t launch_combine_backward_f16(const float* dy, const uint16_t* y_h, const float* y_s,
                                       const int32_t* inv, const float* topk_w, int T, int d,
                                       int k, bool bf16, const uint16_t* ys_h, const float* ys_s,
                                       const float* gate_logit, void* dy_perm, float* dw,
                                       void* dy_shared, float* dgate, hipStream_t s) {
  if (T == 0) return hipSuccess;
#define MOE_CBH(K)                                                                              \
  if (bf16)                                                                                     \
    launch_cbh<K, bf16_t>(dy, y_h, y_s, inv, topk_w, T, d, k, ys_h, ys_s, gate_logit, dy_perm,   \
                          dw, dy_shared, dgate, s);                                             \
  else                                                                                          \
    launch_cbh<K, float>(dy, y_h, y_s, inv, topk_w, T, d, k, ys_h, ys_s, gate_logit, dy_perm, dw, \
                         dy_shared, dgate, s);
  switch (k) {
    case 1: MOE_CBH(1) break;
    case 2: MOE_CBH(2) break;
    case 3: MOE_CBH(3) break;
    case 4: MOE_CBH(4) break;
    case 5: MOE_CBH(5) break;
    case 6: MOE_CBH(6) break;
    case 7: MOE_CBH(7) break;
    case 8: MOE_CBH(8) break;
    default: MOE_CBH(0)
  }
#undef MOE_CBH
  return hipGetLastError();
}

hipError_t launch_unpermute(const float* dx_perm, const int32_t* inv, int T, int d, int k,
                            bool accumulate, float* dx, hipStream_t s) {
  if (T == 0) return hipSuccess;
  switch (k) {
#define MOE_UP(K) case K: launch_up<K>(dx_perm, inv, T, d, accumulate, dx, s); break;
    MOE_UP(1) MOE_UP(2) MOE_UP(3) MOE_UP(4) MOE_UP(5) MOE_UP(6) MOE_UP(7) MOE_UP(8)
#undef MOE_UP
    default:
      hipLaunchKernelGGL(unpermute_any_kernel, dim3(T), dim3(kThreads), 0, s,
                         reinterpret_cast<const f32x4*>(dx_perm), inv, d / 4, k,
                         accumulate ? 1 : 0, reinterpret_cast<f32x4*>(dx));
  }
  return hipGetLastError();
}

hipError_t launch_topk_weights_backward(const float* logits, const int32_t* idx, const float* dw,
                                        int T, int E, int k, bool renorm, float* dL,
                                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int lpt = E <= 8 ? 8 : E <= 16 ? 16 : E <= 32 ? 32 : 64;
  const dim3 grid((unsigned)(((size_t)T * lpt + kThreads - 1) / kThreads));
  const int rn = renorm ? 1 : 0;
  if (lpt == 8)
    hipLaunchKernelGGL(topk_weights_backward_kernel<8>, grid, dim3(kThreads), 0, s, logits, idx, dw, T, E, k, rn, dL);
  else if (lpt == 16)
    hipLaunchKernelGGL(topk_weights_backward_kernel<16>, grid, dim3(kThreads), 0, s, logits, idx, dw, T, E, k, rn, dL);
  else if (lpt == 32)
    hipLaunchKernelGGL(topk_weights_backward_kernel<32>, grid, dim3(kThreads), 0, s, logits, idx, dw, T, E, k, rn, dL);
  else
    hipLaunchKernelGGL(topk_weights_backward_kernel<64>, grid, dim3(kThreads), 0, s, logits, idx, dw, T, E, k, rn, dL);
  return hipGetLastError();
}

// MFMA form (bf16 x): experts per workgroup group (16 NB), and tokens per
// partial chunk: about 1024 workgroups over (column blocks x expert groups x
// token chunks), a multiple of 32 between 32 and 1024
int xtg_mfma_nb(int E) { return E <= 16 ? 1 : E <= 32 ? 2 : 4; }
int xtg_mfma_chunk(int T, int d, int E) {
  const long long blocks = (long long)cdiv(d, XM_COLS) * cdiv(E, 16 * xtg_mfma_nb(E));
  const long long want = (long long)T * blocks / 1024;
  return (int)std::min<long long>(1024, std::max<long long>(XM_K, (want + XM_K - 1) / XM_K * XM_K));
}

// workspace: partials [chunks, d, E] fp32 of whichever form runs (fp32 or
// bf16 x), then the split G (hi, lo: [T, EP] bf16 each) of the bf16 form
size_t linear_partials_bytes(int T, int d, int E) {
  const size_t nc = (size_t)std::max(cdiv(T, xtg_chunk(T, d, E)), cdiv(T, xtg_mfma_chunk(T, d, E)));
  return align_up(nc * (size_t)d * E * sizeof(float), 256);
}
size_t split_g_bytes(int T, int E) {
  return align_up((size_t)T * split_ep(E) * sizeof(bf16_t), 256);
}
size_t linear_backward_workspace_bytes(int T, int d, int E) {
  return linear_partials_bytes(T, d, E) + 2 * split_g_bytes(T, E);
}

template <int NB>
void launch_xtg_mfma(const bf16_t* x, const bf16_t* gh, const bf16_t* gl, int T, int d, int E,
                     float* dW, float* part, hipStream_t s) {
  const int tc = xtg_mfma_chunk(T, d, E);
  const int nc = cdiv(T, tc);
  hipLaunchKernelGGL((xtg_mfma_kernel<NB>), dim3(cdiv(d, XM_COLS), nc, cdiv(E, 16 * NB)),
                     dim3(kThreads), 0, s, x, gh, gl, T, d, E, split_ep(E), tc, part);
  const size_t n = (size_t)d * E;
  hipLaunchKernelGGL(sum_chunks_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, part, nc, n, dW);
}

template <int KS>
void launch_dx_mfma(const bf16_t* gh, const bf16_t* gl, const bf16_t* W, int T, int d, int E,
                    float* dx, hipStream_t s) {
  const dim3 grid(cdiv(d, DM_C), cdiv(T, DM_T));
  const int EP = split_ep(E);
  if (E % 8 == 0 && ((uintptr_t)W & 15) == 0)
    hipLaunchKernelGGL((dx_mfma_kernel<KS, true>), grid, dim3(kThreads), 0, s, gh, gl, W, T, d, E,
                       EP, dx);
  else
    hipLaunchKernelGGL((dx_mfma_kernel<KS, false>), grid, dim3(kThreads), 0, s, gh, gl, W, T, d,
                       E, EP, dx);
}

void launch_linear_bwd_mfma(const void* x, const void* W, const float* G, int T, int d, int E,
                            float* dW, float* dx, void* ws, hipStream_t s) {
  float* part = static_cast<float*>(ws);
  bf16_t* gh = reinterpret_cast<bf16_t*>(static_cast<char*>(ws) + linear_partials_bytes(T, d, E));
  bf16_t* gl = reinterpret_cast<bf16_t*>(reinterpret_cast<char*>(gh) + split_g_bytes(T, E));
  const size_t n = (size_t)T * split_ep(E);
  hipLaunchKernelGGL(split_g_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, G, T, E, split_ep(E), gh, gl);
  if (dW) {
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const int nb = xtg_mfma_nb(E);
    if (nb == 1) launch_xtg_mfma<1>(xb, gh, gl, T, d, E, dW, part, s);
    else if (nb == 2) launch_xtg_mfma<2>(xb, gh, gl, T, d, E, dW, part, s);
    else launch_xtg_mfma<4>(xb, gh, gl, T, d, E, dW, part, s);
  }
  if (dx) {
    const bf16_t* Wb = static_cast<const bf16_t*>(W);
    if (E <= 32) launch_dx_mfma<1>(gh, gl, Wb, T, d, E, dx, s);
    else launch_dx_mfma<2>(gh, gl, Wb, T, d, E, dx, s);
  }
}

template <typename XT, int EB>
void launch_linear_bwd(const void* x, const void* W, const float* G, int T, int d, int E,
                       float* dW, float* dx, void* ws, hipStream_t s) {
  if (dW) {
    const int tc = xtg_chunk(T, d, E);
    const int nc = cdiv(T, tc);
    constexpr int CB = XtgShape<EB>::CB;  // columns per block (= xtg_cols(E))
    float* part = static_cast<float*>(ws);
    hipLaunchKernelGGL((xtg_partial_kernel<XT, EB>), dim3(cdiv(d, CB), nc), dim3(kThreads), 0, s,
                       static_cast<const XT*>(x), G, T, d, E, tc, part);
    const size_t n = (size_t)d * E;
    hipLaunchKernelGGL(sum_chunks_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, part, nc, n, dW);
  }
  if (dx)
    hipLaunchKernelGGL((dx_linear_kernel<XT, EB>), dim3(cdiv(d, DXC), cdiv(T, DXT)), dim3(kThreads),
                       0, s, G, static_cast<const XT*>(W), T, d, E, dx);
}

template <typename XT>
void launch_linear_bwd_e(const void* x, const void* W, const float* G, int T, int d, int E,
                         float* dW, float* dx, void* ws, hipStream_t s) {
  if (E <= 8) launch_linear_bwd<XT, 8>(x, W, G, T, d, E, dW, dx, ws, s);
  else if (E <= 16) launch_linear_bwd<XT, 16>(x, W, G, T, d, E, dW, dx, ws, s);
  else if (E <= 32) launch_linear_bwd<XT, 32>(x, W, G, T, d, E, dW, dx, ws, s);
  else launch_linear_bwd<XT, 64>(x, W, G, T, d, E, dW, dx, ws, s);
}

hipError_t launch_linear_backward(const void* x, const void* W, const float* G, int T, int d,
                                  int E, bool bf16, float* dW, float* db, float* dx, void* ws,
                                  hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    launch_linear_bwd_mfma(x, W, G, T, d, E, dW, dx, ws, s);
  else
    launch_linear_bwd_e<float>(x, W, G, T, d, E, dW, dx, ws, s);
  if (db) hipLaunchKernelGGL(colsum_kernel, dim3(E), dim3(kThreads), 0, s, G, T, E, db);
  return hipGetLastError();
}

}  // namespace moe
