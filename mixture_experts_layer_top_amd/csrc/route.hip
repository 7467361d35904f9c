// Router: logits, softmax top-k selection and weights, one launch, one pass
// over x.
//
// Top-k expert choice per token: DisagMoE technical summary, "2.2 AF-Pipe".
//
// bf16 path.  The logits L = x W_r are a skinny contraction (E <= 256
// columns), bound by reading x from HBM once.  W_r is read in the caller's
// [d, E] layout: a K chunk of its rows is one contiguous block, moved to LDS
// with direct-to-LDS loads and read back with the gfx950 LDS transpose read
// (8 consecutive K values of one expert per lane, the B operand of
// v_mfma_f32_16x16x32_bf16); lanes whose columns lie past E read a zero
// patch, so E must only be a multiple of 8 (other E gather their B operand
// from memory one element at a time: small gates, E = 1 in one load).
// bf16 products are exact in fp32; sums are fp32 in a fixed order.
//
//   route_bf16_kernel: a workgroup of NWV wave64s takes 16 MB tokens and
//     the waves split K into NWV ranges.  Each wave walks its range in
//     chunks of 32 ST K values: the chunk's W_r rows go to the wave's own
//     LDS tile, then all its x fragments (16 token rows x 16 contiguous
//     bytes per lane) are loaded into registers before its first MFMA; the
//     partial logits of the waves are added in wave order, then the bias.
//   route_bf16_sw_kernel (long batches, E <= 16): the waves split tokens
//     instead, so each W_r chunk is loaded once per workgroup; x tiles and
//     W_r chunks stream through an LDS ring with one barrier per stage, and
//     each wave holds its tokens' complete logits.
//   Both walk their K chunks in an order rotated by the workgroup index.
//
// Selection and weights: LPT lanes per token (2 to 16, as many as the
// workgroup's lanes allow), each holding every LPT-th logit.  The j-th pick
// is the best (value desc, index asc) strictly below the (j-1)-th pick in
// that order, so no pick is ever marked; exactly equal logits go to the
// lower index.  A NaN logit is taken as -inf, so every token gets k
// distinct experts in [0, E) whatever its logits.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// x is read once: non-temporal loads, which do not displace cached lines
// (with plain loads every fetched line evicts one, and a dirty victim
// costs a write-back: after a 1 GiB write had filled the caches, routing
// 4096 x 4096 tokens took 19 us with plain loads and 15 us with these)
__device__ __forceinline__ bf16x8 load_x(const bf16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return __builtin_bit_cast(bf16x8, v);
}

struct RouteArgs {
  const void* x;
  const void* W;
  const float* bias;
  int T, d, E, k, renorm;
  int32_t* idx;
  float* w;
  float* logits_out;
};

// Reductions over a part of a DPP row (2, 4, 8 or all 16 lanes): xor 1
// and xor 2 inside each quad, then the half-row mirror (lane i <-> 7 - i in
// each 8-lane half) pairs the two quads of a half and the row mirror
// (i <-> 15 - i) the two halves.  Every step combines two lanes' values with
// a commutative operation, so all lanes of the part end with the
// bitwise-same result.  DPP moves run on the vector ALU; the shuffles they
// replace went through the LDS permute unit.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, x)));
}

// Ordered keys of the selection: (value desc, index asc) as one unsigned
// 64-bit integer, larger = better.  The value's bits map monotonically to
// an unsigned 32-bit integer (negative values: all bits flipped; others:
// sign bit set), the index goes below it as 255 - e (E <= 256).  Every
// valid key is above 0, the key of the padded experts.
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_ordered(uint32_t h) {
  return __builtin_bit_cast(float, (h & 0x80000000u) ? (h & 0x7fffffffu) : ~h);
}

// Reductions over LPT consecutive lanes (LPT a power of two up to 16: the
// steps above taken as far as needed)
template <int LPT>
__device__ __forceinline__ float part_max(float x) {
  if (LPT >= 2) x = fmaxf(x, dpp_f<kDppXor1>(x));
  if (LPT >= 4) x = fmaxf(x, dpp_f<kDppXor2>(x));
  if (LPT >= 8) x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  if (LPT >= 16) x = fmaxf(x, dpp_f<kDppMirror>(x));
  return x;
}
template <int LPT>
__device__ __forceinline__ float part_sum(float x) {
  if (LPT >= 2) x += dpp_f<kDppXor1>(x);
  if (LPT >= 4) x += dpp_f<kDppXor2>(x);
  if (LPT >= 8) x += dpp_f<kDppHalfMirror>(x);
  if (LPT >= 16) x += dpp_f<kDppMirror>(x);
  return x;
}
template <int CTRL>
__device__ __forceinline__ uint64_t key_max_step(uint64_t x) {
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(x >> 32));
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > x ? o : x;
}
template <int LPT>
__device__ __forceinline__ uint64_t part_max_key(uint64_t x) {
  if (LPT >= 2) x = key_max_step<kDppXor1>(x);
  if (LPT >= 4) x = key_max_step<kDppXor2>(x);
  if (LPT >= 8) x = key_max_step<kDppHalfMirror>(x);
  if (LPT >= 16) x = key_max_step<kDppMirror>(x);
  return x;
}

// Softmax top-k over `ntok` logits rows in LDS: LPT lanes per token, each
// holding NV = Ep / LPT of the row's logits in registers (expert q + LPT u
// for lane q); waves take groups of 64 / LPT tokens in turn.  The j-th pick
// is the largest key strictly below the (j-1)-th pick's: a per-lane scan of
// NV keys and a reduction over the token's lanes.  NaN logits are taken as
// -inf for the order and the weights.  For k <= 16, lane q keeps the picks
// j = q, q + LPT, ... and the k picks are written together at the end
// (divided by their sum with renormalisation); larger k writes each pick as
// it is found and divides afterwards.  Callers choose LPT so that the
// workgroup's lanes cover its tokens: fewer lanes per token means fewer
// reduction steps per pick and more tokens at once.
template <int NV, int LPT>
__device__ __forceinline__ void select_and_weigh(const float* ll, int lstride, const RouteArgs& a,
                                                 int t_base, int ntok) {
  static_assert(LPT == 1 || LPT == 2 || LPT == 4 || LPT == 8 || LPT == 16, "lanes per token");
  constexpr int TPW = 64 / LPT;              // tokens per wave and pass
  constexpr int KPL = (16 + LPT - 1) / LPT;  // picks a lane keeps (k <= 16)
  const int lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int q = lane & (LPT - 1);
  const int E = a.E, k = a.k;
  for (int g0 = (threadIdx.x >> 6) * TPW; g0 < ntok; g0 += nwaves * TPW) {
    const int tt = g0 + lane / LPT;
    const int t = t_base + tt;
    const bool live = tt < ntok && t < a.T;
    const float* row = ll + (tt < ntok ? tt : 0) * lstride;
    float v[NV];
    uint64_t key[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = q + LPT * u;
      const float l = (e < E) ? row[e] : -INFINITY;
      v[u] = (l == l) ? l : -INFINITY;  // NaN ranks with -inf
      key[u] = (e < E) ? ((uint64_t)ordered_bits(v[u]) << 32) | (uint32_t)(255 - e) : 0ull;
    }
    // softmax denominator relative to the row max
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < NV; ++u) m = fmaxf(m, v[u]);
    m = part_max<LPT>(m);
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < NV; ++u) sum += (q + LPT * u < E) ? __expf(v[u] - m) : 0.f;
    sum = part_sum<LPT>(sum);

    uint64_t prev = ~0ull;
    float sel = 0.f;
    int my_e[KPL];
    float my_ex[KPL];
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      my_e[s] = 0;
      my_ex[s] = 0.f;
    }
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (key[u] < prev && key[u] > best) best = key[u];
      best = part_max_key<LPT>(best);
      prev = best;
      const int be = 255 - (int)(uint32_t)best;
      const float ex = __expf(from_ordered((uint32_t)(best >> 32)) - m);
      sel += ex;
      if (k <= 16) {
#pragma unroll
        for (int s = 0; s < KPL; ++s)
          if (j == q + LPT * s) {
            my_e[s] = be;
            my_ex[s] = ex;
          }
      } else if (q == 0 && live) {
        a.idx[(size_t)t * k + j] = be;
        a.w[(size_t)t * k + j] = a.renorm ? ex : ex / sum;
      }
    }
    if (k <= 16) {
      if (live) {
#pragma unroll
        for (int s = 0; s < KPL; ++s) {
          const int j = q + LPT * s;
          if (j < k) {
            a.idx[(size_t)t * k + j] = my_e[s];
            a.w[(size_t)t * k + j] = a.renorm ? my_ex[s] / sel : my_ex[s] / sum;
          }
        }
      }
    } else if (a.renorm && q == 0 && live) {
      for (int j = 0; j < k; ++j) a.w[(size_t)t * k + j] = a.w[(size_t)t * k + j] / sel;
    }
  }
}

// Lanes per token for a workgroup of `threads` lanes routing `tokens` tokens
// over Ep (padded) experts: every lane busy where the tokens allow, at most
// 16 (one DPP row) and at most 32 keys per lane.
constexpr int lanes_per_token(int threads, int tokens, int Ep) {
  int l = threads / tokens;
  l = l < 1 ? 1 : (l > 16 ? 16 : l);
  while (Ep / l > 32) l *= 2;  // at most 32 keys per lane
  return l > 16 ? 16 : l;
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

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// One direct-to-LDS load: 64 lanes x 16 bytes from their global addresses
// to the 1 KiB of LDS starting at lds_addr (wave-uniform).  Inline assembly:
// the compiler does not model it, so its completion is waited for
// explicitly (wait_vmcnt_route) before the LDS bytes are read.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "s"(lds_addr)
      : "m0", "memory");  // keeps the chunk's x loads after it (waits count in issue order)
}

// The same for a stream read once (x): the non-temporal form.
__device__ __forceinline__ void dma16_nt(const void* gptr, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off nt"
      :
      : "v"(gptr), "s"(lds_addr)
      : "m0", "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding);
// a compiler memory barrier, so no LDS read moves above it
template <int N>
__device__ __forceinline__ void wait_vmcnt_route() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// LDS bytes of the route kernel: the waves' W_r tiles (KC rows x E columns
// each, plus a 16-byte zero patch), then reused for the partial logits
// [NWV][TW][Ep] and the logits [TW][Ep + 1].
template <int NB, int MB, int NWV, int ST>
struct RouteCfg {
  static constexpr int Ep = NB * 16, TW = MB * 16, KC = 32 * ST;
  static constexpr int WTILE = KC * Ep * 2;                 // bytes, E <= Ep
  static constexpr int ZERO = NWV * WTILE;                  // offset of the zero patch
  static constexpr int W_BYTES = ZERO + 16;
  static constexpr int P_BYTES = NWV * TW * Ep * 4;
  static constexpr int L_BYTES = TW * (Ep + 1) * 4;
  static constexpr int LDS = W_BYTES > P_BYTES ? (W_BYTES > L_BYTES ? W_BYTES : L_BYTES)
                                               : (P_BYTES > L_BYTES ? P_BYTES : L_BYTES);
  static constexpr int WL = ST * NB;  // 16-byte pieces of a W_r chunk per lane (at most)
};

// NB = ceil(E / 16) column blocks of 16 experts; MB = token blocks of 16 per
// workgroup; NWV waves split K; ST MFMA K-steps (of 32) per chunk.
// WTR: E % 8 == 0, W_r staged through LDS; otherwise the B operand is
// gathered from memory one element at a time (small E only: the gate of a
// shared expert has E = 1, whose column is contiguous).
template <int NB, int MB, int NWV, int ST, bool WTR>
__global__ __launch_bounds__(NWV * 64) void route_bf16_kernel(RouteArgs a) {
  using C = RouteCfg<NB, MB, NWV, ST>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int Ep = C::Ep, TW = C::TW, KC = C::KC;
  constexpr int NT = NWV * 64;
  constexpr int ls = Ep + 1;  // LDS row stride of the logits, in floats

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t_base = blockIdx.x * TW;
  const int d = a.d, E = a.E;
  const int kq = cdiv(cdiv(d, NWV), KC) * KC;  // K per wave, whole chunks
  const int kb = min(d, wave * kq), ke = min(d, kb + kq);
  const int nch = cdiv(ke - kb, KC);

  const bf16_t* X = static_cast<const bf16_t*>(a.x);
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  const bf16_t* xr[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = t_base + mb * 16 + (lane & 15);
    xr[mb] = X + (size_t)(t < a.T ? t : 0) * d + (lane >> 4) * 8;  // rows past T read token 0
  }

  // W_r tile of this wave: the chunk's KC rows x E columns as in memory
  char* wt = smem + wave * C::WTILE;
  if (WTR && tid < 4) reinterpret_cast<uint32_t*>(smem + C::ZERO)[tid] = 0u;
  // transpose-read offsets: lane l takes column 16 nb + l % 16 of rows
  // kr .. kr + 3 (and + 4); lanes whose 4 columns lie past E read zeros
  const int kr = (lane >> 4) * 8 + ((lane & 15) >> 2), cq = (lane & 3) * 4;
  const uint32_t zrel = (uint32_t)(C::ZERO - wave * C::WTILE);  // the zero patch, from wt
  uint32_t tr_lo[NB];
  bool tr_in[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = nb * 16 + cq;
    tr_in[nb] = col < E;
    tr_lo[nb] = (uint32_t)((kr * E + col) * 2);
  }

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One chunk: ST K-steps of 32.  Its W_r rows (KC x E bf16, one contiguous
  // block) go straight to the wave's LDS tile with direct-to-LDS loads,
  // issued first; then its x fragments are loaded into registers.  Loads
  // complete in issue order, so the first wait for an x fragment (inserted
  // by the compiler) also covers the W_r rows; an explicit wait for them
  // precedes the transpose reads.  Rows past the wave's range load a valid
  // W_r row and meet zero x fragments.
  const int cbytes = KC * E * 2;                 // bytes of a full W_r chunk
  const int nwl = WTR ? cdiv(cbytes, 1024) : 0;  // 1 KiB loads per chunk
  const uint32_t wt_lds = lds_addr_of(wt);
  const char* Wb = reinterpret_cast<const char*>(W);
  const long long wlast = (long long)d * E * 2 - 16;  // last 16 bytes of W_r
  const bf16x8 zero8 = {};
  if (WTR) __syncthreads();  // the zero patch is written
  // chunk order rotated per workgroup (as in the shared-W_r kernel below):
  // concurrent workgroups then read different offsets of their rows
  const int rot = nch > 0 ? (int)(blockIdx.x % (unsigned)nch) : 0;
  for (int c0 = 0; c0 < nch; ++c0) {
    const int c = c0 + rot < nch ? c0 + rot : c0 + rot - nch;
    const int k0 = kb + c * KC;
    if (WTR) {
      // the wave's earlier transpose reads of its tile have completed
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const long long base = (long long)k0 * E * 2;
      for (int j = 0; j < nwl; ++j) {
        long long off = base + j * 1024 + lane * 16;
        if (off > wlast) off = wlast;
        dma16(Wb + off, wt_lds + (uint32_t)(j * 1024));
      }
    }
    bf16x8 xv[ST][MB];
    if (k0 + KC <= ke) {
#pragma unroll
      for (int st = 0; st < ST; ++st)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xv[st][mb] = load_x(xr[mb] + k0 + st * 32);
    } else {
      // ragged last chunk: K past the wave's range contributes zeros
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        const int kk = k0 + st * 32 + (lane >> 4) * 8;  // d % 8 == 0: 8 values all in or all out
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xv[st][mb] = kk < ke ? load_x(xr[mb] + k0 + st * 32) : zero8;
      }
    }
    if (WTR) {
      // the W_r rows have landed once at most the x loads are outstanding
      if (ST * MB == 1) wait_vmcnt_route<1>();
      else if (ST * MB == 2) wait_vmcnt_route<2>();
      else if (ST * MB == 4) wait_vmcnt_route<4>();
      else if (ST * MB == 8) wait_vmcnt_route<8>();
      else wait_vmcnt_route<16>();
    }
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      bf16x8 bv[NB];
      if (WTR) {
        const uint32_t base = (uint32_t)(st * 32 * E * 2);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t lo_off = tr_in[nb] ? tr_lo[nb] + base : zrel;
          const uint32_t hi_off = tr_in[nb] ? tr_lo[nb] + base + (uint32_t)(4 * E * 2) : zrel;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wt + lo_off));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wt + hi_off));
          bv[nb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      } else {
        // gather: lane l takes expert 16 nb + l % 16, K rows kk .. kk + 7
        const int kk = k0 + st * 32 + (lane >> 4) * 8;
        if (E == 1) {
          // one contiguous column: lane l % 16 == 0 loads its 8 K values at once
          bv[0] = ((lane & 15) == 0 && kk < ke) ? *reinterpret_cast<const bf16x8*>(W + kk) : zero8;
#pragma unroll
          for (int nb = 1; nb < NB; ++nb) bv[nb] = zero8;
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int e = nb * 16 + (lane & 15);
            bf16_t tmp[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
              tmp[i] = (e < E && kk < ke) ? W[(size_t)(kk + i) * E + e] : (bf16_t)0;
            u32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (uint32_t)tmp[2 * i] | ((uint32_t)tmp[2 * i + 1] << 16);
            bv[nb] = as_bf16x8(v);
          }
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[st][mb], bv[nb], acc[mb][nb], 0, 0, 0);
    }
  }
  // partial logits of each wave; the accumulator layout of a 16 x 16 block
  // is column lane % 16, rows 4 (lane / 16) + i
  __syncthreads();  // every wave is done with its W_r tile
  float* part = reinterpret_cast<float*>(smem);  // [NWV][TW][Ep]
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
  float* ll = part;  // [TW][ls] logits
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * NT;
    if (i < TW * Ep) ll[(i / Ep) * ls + (i % Ep)] = lv[u];
  }
  __syncthreads();
  write_logits(ll, ls, a, t_base, TW);
  constexpr int LPT = lanes_per_token(NT, TW, Ep);
  select_and_weigh<Ep / LPT, LPT>(ll, ls, a, t_base, TW);
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
  constexpr int LPT = lanes_per_token(kThreads, kTok, NV * 16);
  select_and_weigh<NV * 16 / LPT, LPT>(ll, ls, a, t_base, kTok);
}

// ------------------------------------------------------------------------
// Long token batches: a workgroup of NWV waves takes 16 NWV tokens (16 per
// wave, each wave the full K), so every K chunk of W_r is loaded once per
// workgroup and shared by all its waves.  Both operands move HBM -> LDS
// with direct-to-LDS loads through a ring of RING stages of KC K values:
// the x tile [16 NWV rows][KC] (one 1 KiB load covers whole 128-byte lines
// of 1024 / (2 KC) token rows, the 16-byte chunk index XOR-ed with (row / 2)
// mod 8 as in the grouped GEMM's A layout), and the W_r rows of the chunk
// [KC][E] as one contiguous block.  Loads are dealt round-robin over the
// waves (a wave re-issues a load already in its list, same bytes to the same
// place, when the count does not divide evenly), each wave waits for its own
// loads of a stage, and a barrier makes the stage visible: one barrier per
// stage.  Each wave then holds its tokens' complete logits: no reduction
// across waves.  Requires d % KC == 0 and E % 8 == 0.
// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 63] (larger n waits for 63)
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
  switch (n) {
#define MOE_W4(b) case b: wait_vmcnt_route<b>(); break; case b + 1: wait_vmcnt_route<b + 1>(); break; \
                  case b + 2: wait_vmcnt_route<b + 2>(); break; case b + 3: wait_vmcnt_route<b + 3>(); break;
    MOE_W4(0) MOE_W4(4) MOE_W4(8) MOE_W4(12) MOE_W4(16) MOE_W4(20) MOE_W4(24) MOE_W4(28)
    MOE_W4(32) MOE_W4(36) MOE_W4(40) MOE_W4(44) MOE_W4(48) MOE_W4(52) MOE_W4(56) MOE_W4(60)
#undef MOE_W4
    default: wait_vmcnt_route<63>(); break;
  }
}

template <int NB, int NWV, int KC, int RING>
struct SwCfg {
  static constexpr int Ep = NB * 16, TB = 16 * NWV;
  static constexpr int X_BYTES = TB * KC * 2;
  static constexpr int W_BYTES = KC * Ep * 2;         // E <= Ep
  static constexpr int STAGE = X_BYTES + W_BYTES;
  static constexpr int ZERO = RING * STAGE;           // 16-byte zero patch
  static constexpr int LDS_RING = ZERO + 16;
  static constexpr int L_BYTES = TB * (Ep + 1) * 4;
  static constexpr int LDS = LDS_RING > L_BYTES ? LDS_RING : L_BYTES;
  static constexpr int XL = X_BYTES / 1024;           // x loads per stage
  static constexpr int CPR = KC / 8;                  // 16-byte chunks per x row
  static constexpr int RPL = 1024 / (KC * 2);         // x rows per load
  static_assert(KC == 64 || KC == 128 || KC == 256 || KC == 512, "chunk");
  static_assert(X_BYTES % 1024 == 0, "x loads");
};

template <int NB, int NWV, int KC, int RING>
__global__ __launch_bounds__(NWV * 64) void route_bf16_sw_kernel(RouteArgs a) {
  using C = SwCfg<NB, NWV, KC, RING>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr int Ep = C::Ep, TB = C::TB, KS = KC / 32;
  constexpr int ls = Ep + 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t_base = blockIdx.x * TB;
  const int d = a.d, E = a.E;
  const int ns = d / KC;                               // stages
  const int wl = (KC * E * 2 + 1023) / 1024;           // W_r loads per stage
  const int nl = C::XL + wl;                           // loads per stage
  const int lpw = (nl + NWV - 1) / NWV;                // loads per wave per stage
  const char* X = static_cast<const char*>(a.x);
  const char* W = static_cast<const char*>(a.W);
  const long long w_last = (long long)d * E * 2 - 16;  // last 16 bytes of W_r
  const uint32_t lds0 = lds_addr_of(smem);
  if (tid < 4) reinterpret_cast<uint32_t*>(smem + C::ZERO)[tid] = 0u;

  // load j of a stage (j < nl): x load j < XL fills x rows RPL j .. + RPL - 1
  // of the tile; W_r load j - XL fills bytes 1024 (j - XL) .. of the chunk.
  // This lane's global byte offset at stage 0 and LDS byte offset in a stage.
  // stage st covers K chunk (st + rot) mod ns: workgroups start at
  // different chunks, so the rows they read at one moment (d * 2 bytes
  // apart) do not all sit at the same offset in their rows, which measured
  // as a strong slowdown of the whole stream (same-offset requests of every
  // compute unit collide in the memory channels)
  const int rot = (int)(blockIdx.x % (unsigned)ns);
  auto issue_stage = [&](int st) {
    const uint32_t slot = lds0 + (uint32_t)((st % RING) * C::STAGE);
    int kc = st + rot;
    if (kc >= ns) kc -= ns;
    for (int i = 0; i < lpw; ++i) {
      int j = wave + i * NWV;
      if (j >= nl) j = j % nl;  // a repeat: same bytes to the same place
      if (j < C::XL) {
        const int row = j * C::RPL + lane / C::CPR;
        const int chunk = (lane % C::CPR) ^ ((row >> 1) & (C::CPR - 1));
        int t = t_base + row;
        if (t >= a.T) t = 0;  // rows past T read token 0; their logits are never stored
        const long long off = ((long long)t * d + (long long)kc * KC + chunk * 8) * 2;
        dma16_nt(X + off, slot + (uint32_t)(j * 1024));
      } else {
        long long off = (long long)kc * KC * E * 2 + (long long)(j - C::XL) * 1024 + lane * 16;
        if (off > w_last) off = w_last;  // past the chunk (last load of a small E): unused bytes
        dma16(W + off, slot + (uint32_t)(C::X_BYTES + (j - C::XL) * 1024));
      }
    }
  };

  // fragment read offsets inside a stage: A = this wave's 16 token rows,
  // K step ks chunk 4 ks + lane / 16 (swizzled); B = W_r rows kr .. kr + 3
  // and + 4, column 16 nb + 4 (lane % 4) (lanes past E read the zero patch)
  const int l15 = lane & 15;
  const int arow = wave * 16 + l15;
  int a_rd[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    a_rd[ks] = arow * KC * 2 + (((ks * 4 + (lane >> 4)) ^ ((arow >> 1) & (C::CPR - 1))) << 4);
  const int kr = (lane >> 4) * 8 + (l15 >> 2), cq = (lane & 3) * 4;
  uint32_t b_rd[NB];
  bool b_in[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    b_in[nb] = nb * 16 + cq < E;
    b_rd[nb] = (uint32_t)(C::X_BYTES + (kr * E + nb * 16 + cq) * 2);
  }

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  __syncthreads();  // the zero patch is written
  for (int st = 0; st < RING - 1 && st < ns; ++st) issue_stage(st);
  for (int st = 0; st < ns; ++st) {
    // this wave's loads of stage st have landed once at most those of the
    // later stages already issued are outstanding
    wait_vmcnt_rt(lpw * min(RING - 2, ns - 1 - st));
    // every wave's part of stage st is visible, and every wave is done
    // reading stage st - 1 (its reads drained before the barrier)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (st + RING - 1 < ns) issue_stage(st + RING - 1);  // into the slot of stage st - 1
    const char* sl = smem + (st % RING) * C::STAGE;
    const uint32_t zrel = (uint32_t)(C::ZERO - (st % RING) * C::STAGE);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(sl + a_rd[ks]);
      const uint32_t kb_off = (uint32_t)(ks * 32 * E * 2);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t lo = b_in[nb] ? b_rd[nb] + kb_off : zrel;
        const uint32_t hi = b_in[nb] ? b_rd[nb] + kb_off + (uint32_t)(4 * E * 2) : zrel;
        const bf16x4 blo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sl + lo));
        const bf16x4 bhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(sl + hi));
        const bf16x8 bv = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[nb], 0, 0, 0);
      }
    }
  }
  wait_vmcnt_route<0>();
  __syncthreads();  // every wave is done with the ring
  // logits of this wave's 16 tokens, plus the bias (column lane % 16, rows
  // 4 (lane / 16) + i of each accumulator block)
  float* ll = reinterpret_cast<float*>(smem);  // [TB][ls]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = wave * 16 + (lane >> 4) * 4 + i;
      const int e = nb * 16 + l15;
      ll[tt * ls + e] = acc[nb][i] + ((a.bias && e < E) ? a.bias[e] : 0.f);
    }
  __syncthreads();
  write_logits(ll, ls, a, t_base, TB);
  constexpr int LPT = lanes_per_token(NWV * 64, TB, Ep);
  select_and_weigh<Ep / LPT, LPT>(ll, ls, a, t_base, TB);
}

// Raise kernel KERN's dynamic LDS limit to `bytes`, once per device: a
// function attribute, not a stream operation, so that later launches (also
// under graph capture) make no host call besides the launch.
constexpr int kMaxDevices = 64;
template <auto KERN>
hipError_t allow_lds(int bytes) {
  static bool done[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool known = dev >= 0 && dev < kMaxDevices;
  if (known && done[dev]) return hipSuccess;
  e = hipFuncSetAttribute((const void*)KERN, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && known) done[dev] = true;
  return e;
}

template <int NB, int NWV, int KC, int RING>
hipError_t launch_sw(const RouteArgs& a, hipStream_t s) {
  using C = SwCfg<NB, NWV, KC, RING>;
  static_assert(C::LDS <= 160 * 1024, "LDS");
  auto kern = route_bf16_sw_kernel<NB, NWV, KC, RING>;
  if (C::LDS > 65536) {
    hipError_t e = allow_lds<route_bf16_sw_kernel<NB, NWV, KC, RING>>(C::LDS);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(cdiv(a.T, C::TB)), dim3(NWV * 64), C::LDS, s, a);
  return hipGetLastError();
}

template <int NB, int MB, int NWV, bool WTR>
hipError_t launch_cfg(const RouteArgs& a, hipStream_t s) {
  // K-steps per chunk: a chunk's x loads (16 KiB a wave at most, 64
  // registers) are all in flight before its first MFMA, and the waves' W_r
  // tiles take at most 64 KiB of LDS
  constexpr int ST_X = 16 / MB < 8 ? 16 / MB : 8;
  constexpr int ST_W = 1024 / (NB * 16 * NWV) > 0 ? 1024 / (NB * 16 * NWV) : 1;
  constexpr int ST = ST_X < ST_W ? ST_X : ST_W;
  using C = RouteCfg<NB, MB, NWV, ST>;
  static_assert(C::LDS <= 160 * 1024, "LDS");
  auto kern = route_bf16_kernel<NB, MB, NWV, ST, WTR>;
  if (C::LDS > 65536) {
    hipError_t e = allow_lds<route_bf16_kernel<NB, MB, NWV, ST, WTR>>(C::LDS);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(cdiv(a.T, C::TW)), dim3(NWV * 64), C::LDS, s, a);
  return hipGetLastError();
}

// Tokens per workgroup (16 MB) and K-splitting waves (NWV): the kernel
// streams x once, so it wants many loads in flight on every compute unit,
// while W_r is re-read (from L2) once per workgroup -- more tokens per
// workgroup means fewer W_r reads per token but fewer workgroups.  E not a
// multiple of 8 (small gates) takes one shape.
template <int NB>
hipError_t launch_nb(const RouteArgs& a, hipStream_t s) {
  // more than 128 experts: 4-wave workgroups (one per SIMD, the whole
  // register file) keep the 16 accumulator blocks and two chunks in registers
  constexpr int NWS = NB >= 8 ? 4 : 8;
  if (a.E % 8 != 0) return launch_cfg<NB, 1, NWS, false>(a, s);
  // long batches with at most 16 experts: the shared-W_r kernel, once it
  // has a workgroup per compute unit (same box, 134 MB of x: 52 -> 49 us at
  // 8 experts; at 64 experts it measured 66 us against this kernel's 64)
  if constexpr (NB == 1) {
    if (a.d % 256 == 0 && cdiv(a.T, 64) >= device_cu_count()) return launch_sw<1, 4, 256, 3>(a, s);
  }
  if constexpr (NB <= 4) {
    if (a.T >= 256 * 64) return launch_cfg<NB, 4, 4, true>(a, s);
    if (a.T >= 256 * 32) return launch_cfg<NB, 2, 4, true>(a, s);
  }
  if (a.T >= 256 * 16 * 2) return launch_cfg<NB, 1, 4, true>(a, s);
  return launch_cfg<NB, 1, NWS, true>(a, s);
}

}  // namespace

hipError_t launch_route(const void* x, const void* W_r, const float* bias, int T, int d, int E,
                        int k, bool renorm, bool bf16, int32_t* idx, float* w, float* logits_out,
                        hipStream_t s) {
  RouteArgs a{x, W_r, bias, T, d, E, k, renorm ? 1 : 0, idx, w, logits_out};
  if (!bf16) {
    const size_t lds = (size_t)64 * (E + 1) * 4;  // <= 64 * 257 * 4 = 65792 bytes
    auto launch = [&](auto kern) -> hipError_t {
      hipLaunchKernelGGL(kern, dim3(cdiv(T, 64)), dim3(kThreads), lds, s, a);
      return hipGetLastError();
    };
    // logits per lane in the selection: E / 16 rounded up (only the widest
    // form can need more than 64 KiB of LDS: E = 256)
    if (E <= 16) return launch(route_f32_kernel<1>);
    if (E <= 32) return launch(route_f32_kernel<2>);
    if (E <= 64) return launch(route_f32_kernel<4>);
    if (lds > 65536) {
      hipError_t e = allow_lds<route_f32_kernel<16>>(64 * 257 * 4);
      if (e != hipSuccess) return e;
    }
    return launch(route_f32_kernel<16>);
  }
  // column blocks of 16 experts, rounded up to one of a few widths (the
  // columns past E read zeros and are never selected)
  const int nb = cdiv(E, 16);
  if (nb <= 1) return launch_nb<1>(a, s);
  if (nb <= 2) return launch_nb<2>(a, s);
  if (nb <= 4) return launch_nb<4>(a, s);
  if (nb <= 8) return launch_nb<8>(a, s);
  return launch_nb<16>(a, s);
}

}  // namespace moe
