// Dispatch: per-expert histogram, exclusive prefix scan, stable permutation
// and (optionally) the gather of token rows into expert-major order.
//
// Dispatch of each token to its k experts: DisagMoE technical summary,
// "2.2 AF-Pipe"; fetching the tokens an expert needs: COMET page, "COMET's
// Technical Principles" (computation rescheduling).
//
// The row order is fixed (stable counting sort): expert-major, tokens
// ascending inside an expert.  No atomic decides an order, so the result is
// deterministic:
//   1. hist:  each block of 256 tokens counts its (t, j) pairs per expert
//             in LDS and writes its block histogram;
//   2. scan:  the per-expert totals become the offsets, and the block
//             histograms each block's first row per expert;
//   3. rank:  each block marks its tokens in per-expert bit columns (LDS
//             OR) and ranks each pair by popcounts of the bits below it;
//   4. gather (optional): x_perm[r] = x[perm_token[r]], 16-byte vectors.
// A batch of at most 4096 tokens and 8192 (token, expert) pairs is permuted
// in one launch: all of its bit columns fit in every workgroup's LDS, and
// every workgroup builds them (measured: the two-launch path's 10.9 µs
// become 6.7 µs at T = 128, and about 12 µs stay about 12 µs at T = 4096,
// E = 8, k = 2).  Otherwise, when the block histograms
// are small (blocks x experts <= 32768), every rank block does the scan
// itself (its own column prefixes, and the totals): two launches, hist and
// scan+rank.  Otherwise hist also adds into the global counts (integer adds
// commute) and one workgroup scans.
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kPT = 256;       // tokens per block in hist / rank
constexpr int kThreads = 256;
constexpr int kKR = 8;         // picks of a token held in registers

// The first min(k, kKR) picks of one token, all loads issued before any is
// used (addresses clamped to the token's row, so no predicates).
__device__ __forceinline__ void load_picks(const int32_t* __restrict__ it, int k, int (&er)[kKR]) {
#pragma unroll
  for (int j = 0; j < kKR; ++j) er[j] = it[min(j, k - 1)];
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Block histogram over kPT = 256 tokens (thread i = token t0 + i): the same
// per-expert token bit columns as the rank kernel, so counts and ranks
// agree by construction (an expert repeated in one token's list counts
// once there and in the ranks).
__global__ __launch_bounds__(kThreads) void hist_kernel(const int32_t* __restrict__ idx, int T,
                                                        int E, int k, int32_t* __restrict__ blk_cnt,
                                                        int32_t* __restrict__ counts) {
  constexpr int NWD = kPT / 64;
  __shared__ unsigned long long bits[256 * NWD];  // [E][NWD]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < E * NWD; i += kThreads) bits[i] = 0ull;
  __syncthreads();
  const int t = blockIdx.x * kPT + tid;
  if (t < T) {
    const int32_t* it = idx + (size_t)t * k;
    int er[kKR];
    load_picks(it, k, er);
#pragma unroll
    for (int j = 0; j < kKR; ++j)
      if (j < k) atomicOr(&bits[er[j] * NWD + wave], 1ull << lane);
    for (int j = kKR; j < k; ++j) atomicOr(&bits[it[j] * NWD + wave], 1ull << lane);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < NWD; ++w) c += __popcll(bits[e * NWD + w]);
    blk_cnt[(size_t)blockIdx.x * E + e] = c;
    if (counts && c) atomicAdd(&counts[e], c);
  }
}

// One workgroup of 1024 threads.  Thread (part, e) owns a contiguous range
// of blocks for expert e; part totals are scanned in LDS.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts, int E,
                                                    int nb, const int32_t* __restrict__ blk_cnt,
                                                    int32_t* __restrict__ blk_base,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int off[257];
  __shared__ int part_sum[1024];
  const int tid = threadIdx.x;
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = run;
      run += counts[e];
    }
    off[E] = run;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) offsets[e] = off[e];

  const int P = max(1, 1024 / E);  // parts per expert
  const int e = tid % E, part = tid / E;
  const bool active = part < P;
  const int b_lo = active ? (int)((long long)nb * part / P) : 0;
  const int b_hi = active ? (int)((long long)nb * (part + 1) / P) : 0;
  int sum = 0;
  for (int b = b_lo; b < b_hi; ++b) sum += blk_cnt[(size_t)b * E + e];
  part_sum[tid] = sum;
  __syncthreads();
  if (active) {
    int run = off[e];
    for (int p2 = 0; p2 < part; ++p2) run += part_sum[p2 * E + e];
    for (int b = b_lo; b < b_hi; ++b) {
      blk_base[(size_t)b * E + e] = run;
      run += blk_cnt[(size_t)b * E + e];
    }
  }
}

// This block's first row per expert (sbase, LDS) from the block histograms
// blk_cnt [nb, E]: offsets (exclusive scan of the per-expert totals) plus
// the counts of the earlier blocks.  Block 0 also writes counts and offsets.
__device__ __forceinline__ void block_bases(const int32_t* __restrict__ blk_cnt, int nb, int E,
                                            int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets, int* sbase) {
  __shared__ int psum[kThreads], ppre[kThreads], wsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = max(1, kThreads / E);  // parts per expert column (E <= 256)
  const int e = tid % E, part = tid / E;
  int s_all = 0, s_pre = 0;
  if (part < P) {
    const int b_lo = (int)((long long)nb * part / P), b_hi = (int)((long long)nb * (part + 1) / P);
    // 8 loads in flight at a time (clamped addresses; entries past b_hi count 0)
    for (int b0 = b_lo; b0 < b_hi; b0 += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = blk_cnt[(size_t)min(b0 + u, b_hi - 1) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = b0 + u;
        const int v = b < b_hi ? c[u] : 0;
        s_all += v;
        if (b < (int)blockIdx.x) s_pre += v;
      }
    }
  }
  psum[tid] = s_all;
  ppre[tid] = s_pre;
  __syncthreads();
  int tot = 0, pre = 0;
  if (tid < E) {
    for (int q = 0; q < P; ++q) {
      tot += psum[q * E + tid];
      pre += ppre[q * E + tid];
    }
  }
  // exclusive scan of the totals over experts: wave prefix, then wave sums
  int incl = wave_incl_sum(tot);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  for (int w2 = 0; w2 < wave; ++w2) incl += wsum[w2];
  const int excl = incl - tot;
  if (tid < E) {
    sbase[tid] = excl + pre;
    if (blockIdx.x == 0) {
      counts[tid] = tot;
      offsets[tid] = excl;
      if (tid == E - 1) offsets[E] = incl;
    }
  }
}

// Stable ranks of one block of kPT = 256 tokens (thread i = token t0 + i).
// Each token sets its bit in the bit column of every expert it picked
// (LDS OR: the result does not depend on the order of the ORs); a pair's
// row is then base[e] + (rows of e among the block's earlier 64-token
// words) + (bits of e below the token in its own word).  No two pairs of
// one token share an expert, so token order is a total order per expert.
// FUSED: derive the block bases here (block_bases) instead of reading them
// from the scan kernel's blk_base.
template <bool FUSED>
__global__ __launch_bounds__(kThreads) void rank_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ topk_w, int T, int E, int k,
    const int32_t* __restrict__ blk_base, int32_t* __restrict__ perm_token,
    int32_t* __restrict__ inv, float* __restrict__ perm_w, const int32_t* __restrict__ blk_cnt,
    int nb, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  static_assert(kPT == kThreads && kPT % 64 == 0, "one token per thread");
  constexpr int NWD = kPT / 64;                    // 64-token words per expert column
  __shared__ unsigned long long bits[256 * NWD];   // [E][NWD]
  __shared__ int wbase[256 * NWD];                 // [E][NWD]
  __shared__ int sbase[256];                       // FUSED: this block's first row per expert
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < E * NWD; i += kThreads) bits[i] = 0ull;
  if (FUSED) block_bases(blk_cnt, nb, E, counts, offsets, sbase);
  __syncthreads();
  const int t = blockIdx.x * kPT + tid;
  const bool valid = t < T;
  const int32_t* it = idx + (size_t)(valid ? t : 0) * k;
  const unsigned long long me = 1ull << lane;
  int er[kKR];
  if (valid) {
    load_picks(it, k, er);
#pragma unroll
    for (int j = 0; j < kKR; ++j)
      if (j < k) atomicOr(&bits[er[j] * NWD + wave], me);
    for (int j = kKR; j < k; ++j) atomicOr(&bits[it[j] * NWD + wave], me);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < NWD; ++w) {
      wbase[e * NWD + w] = run;
      run += __popcll(bits[e * NWD + w]);
    }
  }
  __syncthreads();
  if (!valid) return;
  const int* base = FUSED ? sbase : blk_base + (size_t)blockIdx.x * E;
  const unsigned long long below = me - 1ull;
  auto place = [&](int j, int e) {
    const int r = base[e] + wbase[e * NWD + wave] + __popcll(bits[e * NWD + wave] & below);
    const size_t pg = (size_t)t * k + j;
    perm_token[r] = t;
    inv[pg] = r;
    if (perm_w) perm_w[r] = topk_w[pg];
  };
#pragma unroll
  for (int j = 0; j < kKR; ++j)
    if (j < k) place(j, er[j]);
  for (int j = kKR; j < k; ++j) place(j, it[j]);
}

// The whole permutation of a short batch in one launch (T <= kSmallT,
// T k <= 2 kSmallT, E * ceil(T / 64) <= kSmallWords): every workgroup
// builds the bit columns of all T tokens in LDS (the same bits as hist and
// rank: a few kilobytes of picks, read from L2), scans them, and places the
// pairs of its own 256 tokens; workgroup 0 also writes counts and offsets.  One launch replaces
// two, and the scattered row writes stay spread over as many compute units
// as before.  Thread i builds from tokens i, i + 1024, ...; each expert's
// column prefix (over its 64-token words) is a wave scan, and the expert
// offsets a scan over the column totals.  Counts, offsets and ranks are
// those of the two-launch path (the same popcounts of the same bits).
constexpr int kSmallT = 4096;
constexpr int kSmallWords = 8192;
constexpr int kSmallThreads = 1024;
__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ topk_w, int T, int E, int k,
    int32_t* __restrict__ perm_token, int32_t* __restrict__ inv, float* __restrict__ perm_w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ unsigned long long bits[kSmallWords];  // [E][NW]
  __shared__ int wbase[kSmallWords];                // [E][NW]: rows of e in earlier words
  __shared__ int ebase[257];                        // offsets
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NWV = kSmallThreads / 64;
  const int NW = cdiv(T, 64);
  for (int i = tid; i < E * NW; i += kSmallThreads) bits[i] = 0ull;
  __syncthreads();
  constexpr int TPT = kSmallT / kSmallThreads;  // tokens per thread
  int er[TPT][kKR];
  // the first min(k, kKR) picks of each of the thread's tokens, all loads
  // issued before any is used (k is uniform: the tests are scalar branches)
#pragma unroll
  for (int q = 0; q < TPT; ++q) {
    const int t = q * kSmallThreads + tid;
    if (t < T) {
#pragma unroll
      for (int j = 0; j < kKR; ++j)
        if (j < k) er[q][j] = idx[(size_t)t * k + j];
    }
  }
#pragma unroll
  for (int q = 0; q < TPT; ++q) {
    const int t = q * kSmallThreads + tid;
    if (t >= T) continue;
    const int w = t >> 6;
    const unsigned long long me = 1ull << (t & 63);
#pragma unroll
    for (int j = 0; j < kKR; ++j)
      if (j < k) atomicOr(&bits[er[q][j] * NW + w], me);
    for (int j = kKR; j < k; ++j) atomicOr(&bits[idx[(size_t)t * k + j] * NW + w], me);
  }
  __syncthreads();
  // column prefixes: wave v scans experts v, v + NWV, ... (lane = word, NW <= 64)
  for (int e = wave; e < E; e += NWV) {
    const int c = lane < NW ? __popcll(bits[e * NW + lane]) : 0;
    const int incl = wave_incl_sum(c);
    if (lane < NW) wbase[e * NW + lane] = incl - c;
    if (lane == 63) ebase[e] = incl;  // the column total, for now
  }
  __syncthreads();
  // offsets: exclusive scan of the totals over experts (wave 0, 4 per lane)
  if (wave == 0) {
    int tot[4], s4 = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = lane * 4 + u;
      tot[u] = e < E ? ebase[e] : 0;
      s4 += tot[u];
    }
    const int incl = wave_incl_sum(s4);
    int run = incl - s4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = lane * 4 + u;
      if (e < E) {
        if (blockIdx.x == 0) {
          counts[e] = tot[u];
          offsets[e] = run;
        }
        ebase[e] = run;
      }
      run += tot[u];
    }
    if (lane == 63 && blockIdx.x == 0) offsets[E] = incl;
  }
  __syncthreads();
  // this workgroup's 256 tokens t0 .. t0 + 255 were built by threads
  // t0 % 1024 .. + 255 from their register slot q = t0 / 1024; those threads
  // place the tokens' pairs
  const int t0 = blockIdx.x * kPT;
  const int q_own = t0 / kSmallThreads;
  const int t = q_own * kSmallThreads + tid;
  if (tid - t0 % kSmallThreads < 0 || tid - t0 % kSmallThreads >= kPT || t >= T) return;
  const int w = t >> 6;
  const unsigned long long below = (1ull << (t & 63)) - 1ull;
  auto place = [&](int j, int e) {
    const int r = ebase[e] + wbase[e * NW + w] + __popcll(bits[e * NW + w] & below);
    const size_t pg = (size_t)t * k + j;
    perm_token[r] = t;
    inv[pg] = r;
    if (perm_w) perm_w[r] = topk_w[pg];
  };
#pragma unroll
  for (int j = 0; j < kKR; ++j) {
    if (j < k) {
      // er[q_own][j] without a run-time register index
      int e = er[0][j];
#pragma unroll
      for (int q = 1; q < TPT; ++q)
        if (q == q_own) e = er[q][j];
      place(j, e);
    }
  }
  for (int j = kKR; j < k; ++j) place(j, idx[(size_t)t * k + j]);
}

// x_perm[r, :] = x[perm_token[r], :] for the rows r < offsets[E] the rank
// kernel wrote (all T k of them unless a token listed an expert twice);
// rows of `vecs` 16-byte vectors.  A block copies 8 rows; a thread takes
// columns c, c + 256, ... of all 8 and issues the 8 loads of a column
// before its stores (rows past the end re-read the block's first source row
// and are not stored), so 8 loads are in flight per thread instead of one
// load-store round trip at a time.
constexpr int kGatherRows = 8;
__global__ __launch_bounds__(kThreads) void gather_kernel(const u32x4* __restrict__ x,
                                                          const int32_t* __restrict__ perm_token,
                                                          const int32_t* __restrict__ offsets,
                                                          int E, int vecs,
                                                          u32x4* __restrict__ x_perm) {
  const int R = offsets[E];
  const int r0 = blockIdx.x * kGatherRows;
  if (r0 >= R) return;
  const int nr = min(kGatherRows, R - r0);
  size_t src[kGatherRows];
#pragma unroll
  for (int j = 0; j < kGatherRows; ++j)
    src[j] = (size_t)perm_token[r0 + (j < nr ? j : 0)] * vecs;
  for (int c = threadIdx.x; c < vecs; c += kThreads) {
    u32x4 v[kGatherRows];
#pragma unroll
    for (int j = 0; j < kGatherRows; ++j) v[j] = x[src[j] + c];
#pragma unroll
    for (int j = 0; j < kGatherRows; ++j)
      if (j < nr) x_perm[(size_t)(r0 + j) * vecs + c] = v[j];
  }
}

}  // namespace

// Static scratch of the allocation-free permute: each device holds its own
// copy of this array (until the process ends).  Host code never uses its
// name as an address: the device address comes from hipGetSymbolAddress,
// once per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};  // per device
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t permute_workspace_bytes(int T, int E, int k) {
  (void)k;
  const size_t nb = (size_t)cdiv(T, kPT);
  return 2 * align_up(nb * E * sizeof(int32_t), 256);
}

hipError_t launch_permute(const int32_t* idx, const float* topk_w, const void* x, int T, int d,
                          int E, int k, bool bf16, int32_t* counts, int32_t* offsets,
                          int32_t* perm_token, int32_t* inv, float* perm_w, void* x_perm,
                          void* ws, hipStream_t s) {
  const int nb = cdiv(T, kPT);
  int32_t* blk_cnt = static_cast<int32_t*>(ws);
  int32_t* blk_base = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                                 align_up((size_t)nb * E * sizeof(int32_t), 256));
  if (T <= kSmallT && (long long)T * k <= kSmallT * 2 && E * cdiv(T, 64) <= kSmallWords) {
    // one launch: every workgroup builds and scans the whole batch's bit
    // columns and places its own tokens
    hipLaunchKernelGGL(permute_small_kernel, dim3(max(nb, 1)), dim3(kSmallThreads), 0, s, idx,
                       topk_w, T, E, k, perm_token, inv, perm_w, counts, offsets);
  } else if (nb > 0 && (long long)nb * E <= 32768) {
    // two launches: block histograms, then scan + rank in every block
    hipLaunchKernelGGL(hist_kernel, dim3(nb), dim3(kThreads), 0, s, idx, T, E, k, blk_cnt,
                       (int32_t*)nullptr);
    hipLaunchKernelGGL(rank_kernel<true>, dim3(nb), dim3(kThreads), 0, s, idx, topk_w, T, E, k,
                       (const int32_t*)nullptr, perm_token, inv, perm_w, blk_cnt, nb, counts,
                       offsets);
  } else {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(cdiv(E, 256)), dim3(256), 0, s, counts, E);
    if (nb > 0)
      hipLaunchKernelGGL(hist_kernel, dim3(nb), dim3(kThreads), 0, s, idx, T, E, k, blk_cnt,
                         counts);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, counts, E, nb, blk_cnt, blk_base,
                       offsets);
    if (nb > 0)
      hipLaunchKernelGGL(rank_kernel<false>, dim3(nb), dim3(kThreads), 0, s, idx, topk_w, T, E,
                         k, blk_base, perm_token, inv, perm_w, (const int32_t*)nullptr, 0,
                         (int32_t*)nullptr, (int32_t*)nullptr);
  }
  const int R = T * k;
  if (x_perm && R > 0) {
    const int vecs = d * (bf16 ? 2 : 4) / 16;
    hipLaunchKernelGGL(gather_kernel, dim3(cdiv(R, kGatherRows)), dim3(kThreads), 0, s,
                       static_cast<const u32x4*>(x), perm_token, offsets, E, vecs,
                       static_cast<u32x4*>(x_perm));
  }
  return hipGetLastError();
}

}  // namespace moe
