// Grouped expert GEMMs: "layer 0" (gate/up projections with fused SwiGLU)
// and "layer 1" (down projection with optional fused weighted combine).
//
// The two GEMMs of an expert and their decomposition: COMET page, "COMET's
// Technical Principles" -- layer 0 split along the token dimension M,
// layer 1 along the hidden dimension N.  On one GPU that survives as the
// tile walk: layer-0 tiles of one (expert, weight panel) are consecutive
// along M, so the panel is fetched once and reused from L2; layer-1 tiles
// of one (expert, row block) are consecutive along N, so its row block is
// reused and each finished output tile goes straight to the combine.
//
// bf16 kernel (gfx950):
//   * workgroup = 4 wave64s (2 x 2), macro tile 256 rows x 256 accumulator
//     columns; each wave owns 128 x 128 = 8 x 8 blocks of 16 x 16 computed
//     with v_mfma_f32_16x16x32_bf16 (fp32 accumulation);
//   * layer 0: the 256 columns are 128 columns of W_gate and the same 128
//     columns of W_up, so SiLU(h) * u is formed in registers (the two
//     accumulators of an output element sit in the same lane);
//   * K steps of 64, double-buffered in LDS (2 x 64 KiB), one barrier per
//     step; global loads of step i+1 are in flight while step i computes;
//   * A (tokens, K contiguous) is stored row-major with the 16-byte chunk
//     index XOR-swizzled by the row, read with ds_read_b128;
//   * B (weights [K, N], N contiguous) is stored as is, swizzled by 32-byte
//     pairs, and read with ds_read_b64_tr_b16, the gfx950 LDS transpose
//     read, which gives each lane 4 consecutive K values of one column --
//     no repacking of the caller's weights;
//   * rows of layer 0 are gathered on load through the permutation
//     (gather_idx), so the permuted copy of x need not exist;
//   * tiles never straddle experts; each workgroup derives its (expert,
//     tile) from the device-side offsets with a wave prefix sum, so the
//     host never reads the per-expert counts; the workgroup id is remapped
//     so that consecutive tiles land on the same XCD (and its L2).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 256;        // rows per tile
constexpr int BNA = 256;       // accumulator columns per tile
constexpr int BK = 64;         // K per pipeline step
constexpr int kThreads = 256;  // 4 waves
constexpr int A_ELEMS = BM * BK;    // 16384 bf16 = 32 KiB
constexpr int B_ELEMS = BK * BNA;   // 16384 bf16 = 32 KiB
constexpr int STAGE = A_ELEMS + B_ELEMS;

struct GemmArgs {
  const bf16_t* A;          // [n_a, K] rows (x for layer 0, activations for layer 1)
  const int32_t* gather;    // row r reads A[gather[r]] (layer 0) or NULL
  const int32_t* offsets;   // [E+1]
  int E, rows, K, N;
  const bf16_t* B0;         // [E, K, N]: W_gate (layer 0) or W_down (layer 1)
  const bf16_t* B1;         // [E, K, N]: W_up (layer 0) or NULL
  bf16_t* a_out;            // layer 0 output [rows, N]
  float* y_perm;            // layer 1 output [rows, N] or NULL
  const int32_t* scatter;   // layer 1 fused combine target row, or NULL (identity)
  const float* row_w;       // layer 1 fused combine weight, or NULL (1)
  float* y;                 // layer 1 fused combine target, or NULL
  int tiles_n;              // column tiles per expert
  int grid_per_xcd;         // padded grid / 8
};

struct TileInfo {
  int e, row0, row_end, n_t, m_t;
  bool ok;
};

// Map a logical tile id to (expert, m-tile, n-tile).  Every wave computes the
// same answer independently from offsets (E <= 256: 4 experts per lane).
template <bool M_ORDERED>
__device__ __forceinline__ TileInfo locate_tile(const GemmArgs& p, int tile) {
  const int lane = threadIdx.x & 63;
  int cnt_tiles[4], mt[4], offe[4];
  int lane_sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane * 4 + u;
    int m = 0, o = 0;
    if (e < p.E) {
      o = p.offsets[e];
      m = cdiv(p.offsets[e + 1] - o, BM);
    }
    mt[u] = m;
    offe[u] = o;
    cnt_tiles[u] = m * p.tiles_n;
    lane_sum += cnt_tiles[u];
  }
  // inclusive wave prefix of lane_sum
  int incl = lane_sum;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int v = __shfl_up(incl, s);
    if (lane >= s) incl += v;
  }
  int start = incl - lane_sum;
  int hit_e = -1, hit_start = 0, hit_mt = 0, hit_off = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (tile >= start && tile < start + cnt_tiles[u]) {
      hit_e = lane * 4 + u;
      hit_start = start;
      hit_mt = mt[u];
      hit_off = offe[u];
    }
    start += cnt_tiles[u];
  }
  const uint64_t hit = __ballot(hit_e >= 0);
  TileInfo ti;
  ti.ok = hit != 0;
  if (!ti.ok) return ti;
  const int src = __ffsll((unsigned long long)hit) - 1;
  ti.e = __shfl(hit_e, src);
  const int tstart = __shfl(hit_start, src);
  const int tmt = __shfl(hit_mt, src);
  const int toff = __shfl(hit_off, src);
  const int local = tile - tstart;
  if (M_ORDERED) {
    ti.n_t = local / tmt;
    ti.m_t = local - ti.n_t * tmt;
  } else {
    ti.m_t = local / p.tiles_n;
    ti.n_t = local - ti.m_t * p.tiles_n;
  }
  ti.row0 = toff + ti.m_t * BM;
  ti.row_end = min(ti.row0 + BM, p.offsets[ti.e + 1]);
  return ti;
}

// LDS element offsets (bf16 units) of the swizzled layouts
__device__ __forceinline__ int a_lds_off(int row, int chunk) {  // chunk: 16 B, 0..7
  return row * BK + ((chunk ^ (row & 7)) << 3);
}
__device__ __forceinline__ int b_lds_off(int krow, int col) {  // col: bf16 index, 0..255
  const int chunk = col >> 3;
  return krow * BNA + ((chunk ^ ((krow & 15) << 1)) << 3) + (col & 7);
}

template <bool UP>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * STAGE];

  const int b = blockIdx.x;
  const int tile = (b & 7) * p.grid_per_xcd + (b >> 3);
  const TileInfo ti = locate_tile<UP>(p, tile);
  if (!ti.ok) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = p.K, N = p.N;
  const int n0 = ti.n_t * (UP ? BNA / 2 : BNA);

  // ---- global -> LDS loader setup
  // A: thread owns chunk (tid & 7) of rows (tid >> 3) + 32 i
  const int a_chunk = tid & 7;
  const bf16_t* a_src[8];
  bool a_ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = ti.row0 + (tid >> 3) + 32 * i;
    a_ok[i] = r < ti.row_end;
    const int src_row = a_ok[i] ? (p.gather ? p.gather[r] : r) : 0;
    a_src[i] = p.A + (size_t)src_row * K + a_chunk * 8;
  }
  // B: thread owns chunk (tid & 31) of K rows (tid >> 5) + 8 i
  const int b_chunk = tid & 31;
  const int b_row = tid >> 5;
  int b_col;
  const bf16_t* bmat;
  if (UP) {
    bmat = (b_chunk < 16) ? p.B0 : p.B1;
    b_col = n0 + (b_chunk & 15) * 8;
  } else {
    bmat = p.B0;
    b_col = n0 + b_chunk * 8;
  }
  const bool b_col_ok = b_col < N;
  const bf16_t* b_src = bmat + (size_t)ti.e * K * N + (size_t)b_row * N + (b_col_ok ? b_col : 0);

  u32x4 ra[8], rb[8];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = a_ok[i] && (k0 + a_chunk * 8 < K);
      ra[i] = ok ? *reinterpret_cast<const u32x4*>(a_src[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = b_col_ok && (k0 + b_row + 8 * i < K);
      rb[i] = ok ? *reinterpret_cast<const u32x4*>(b_src + (size_t)(k0 + 8 * i) * N)
                 : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_lds = [&](int stage) {
    bf16_t* As = lds + stage * STAGE;
    bf16_t* Bs = As + A_ELEMS;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(As + a_lds_off((tid >> 3) + 32 * i, a_chunk)) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(Bs + b_lds_off(b_row + 8 * i, b_chunk * 8)) = rb[i];
  };

  // ---- per-lane LDS read offsets
  int a_rd[8][2];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      a_rd[mi][ks] = a_lds_off(wm * 128 + mi * 16 + (lane & 15), ks * 4 + (lane >> 4));
  int b_col_l[8];
#pragma unroll
  for (int nj = 0; nj < 8; ++nj) {
    int c0;
    if (UP) c0 = (nj < 4) ? (wn * 64 + nj * 16) : (128 + wn * 64 + (nj - 4) * 16);
    else c0 = wn * 128 + nj * 16;
    b_col_l[nj] = c0 + (lane & 3) * 4;
  }
  const int b_krow = (lane >> 4) * 8 + ((lane & 15) >> 2);

  f32x4 acc[8][8];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int nj = 0; nj < 8; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = cdiv(K, BK);
  load_global(0);
  store_lds(0);
  __syncthreads();

  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const bf16_t* As = lds + stage * STAGE;
    const bf16_t* Bs = As + A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[8], bfr[8];
#pragma unroll
      for (int mi = 0; mi < 8; ++mi) af[mi] = *reinterpret_cast<const bf16x8*>(As + a_rd[mi][ks]);
#pragma unroll
      for (int nj = 0; nj < 8; ++nj) {
        const int kr = ks * 32 + b_krow;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(Bs + b_lds_off(kr, b_col_l[nj])));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(Bs + b_lds_off(kr + 4, b_col_l[nj])));
        bfr[nj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int nj = 0; nj < 8; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[nj], acc[mi][nj], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Accumulator layout of a 16 x 16 block: column lane % 16,
  // rows 4 * (lane / 16) + i.
  const int col_l = lane & 15;
  const int row_l = (lane >> 4) * 4;
  if (UP) {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = ti.row0 + wm * 128 + mi * 16 + row_l + i;
        if (row >= ti.row_end) continue;
        bf16_t* orow = p.a_out + (size_t)row * N;
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
          const int col = n0 + wn * 64 + nj * 16 + col_l;
          if (col < N) orow[col] = f32_to_bf16(silu(acc[mi][nj][i]) * acc[mi][nj + 4][i]);
        }
      }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = ti.row0 + wm * 128 + mi * 16 + row_l + i;
        if (row >= ti.row_end) continue;
        float* prow = p.y_perm ? p.y_perm + (size_t)row * N : nullptr;
        float* yrow = nullptr;
        float wgt = 1.f;
        if (p.y) {
          const int tgt = p.scatter ? p.scatter[row] : row;
          yrow = p.y + (size_t)tgt * N;
          if (p.row_w) wgt = p.row_w[row];
        }
#pragma unroll
        for (int nj = 0; nj < 8; ++nj) {
          const int col = n0 + wn * 128 + nj * 16 + col_l;
          if (col >= N) continue;
          const float v = acc[mi][nj][i];
          if (prow) prow[col] = v;
          if (yrow) unsafeAtomicAdd(yrow + col, wgt * v);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// fp32 path (small layers): one thread per output element, sequential FMA.
// ------------------------------------------------------------------------

__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E;  // find e with offsets[e] <= r < offsets[e+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void up_f32_kernel(const float* __restrict__ x, const int32_t* __restrict__ gather,
                              const int32_t* __restrict__ offsets, int E, int rows, int d, int f,
                              const float* __restrict__ Wg, const float* __restrict__ Wu,
                              float* __restrict__ a_out) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * f) return;
  const int r = (int)(i / f), c = (int)(i - (size_t)r * f);
  const int e = expert_of_row(offsets, E, r);
  const float* z = x + (size_t)(gather ? gather[r] : r) * d;
  const float* g = Wg + (size_t)e * d * f + c;
  const float* u = Wu + (size_t)e * d * f + c;
  float h = 0.f, v = 0.f;
  for (int kk = 0; kk < d; ++kk) {
    h = fmaf(z[kk], g[(size_t)kk * f], h);
    v = fmaf(z[kk], u[(size_t)kk * f], v);
  }
  a_out[i] = silu(h) * v;
}

__global__ void down_f32_kernel(const float* __restrict__ a, const int32_t* __restrict__ offsets,
                                int E, int rows, int f, int d, const float* __restrict__ Wd,
                                float* y_perm, const int32_t* __restrict__ scatter,
                                const float* __restrict__ row_w, float* y) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * d) return;
  const int r = (int)(i / d), c = (int)(i - (size_t)r * d);
  const int e = expert_of_row(offsets, E, r);
  const float* ar = a + (size_t)r * f;
  const float* w = Wd + (size_t)e * f * d + c;
  float acc = 0.f;
  for (int kk = 0; kk < f; ++kk) acc = fmaf(ar[kk], w[(size_t)kk * d], acc);
  if (y_perm) y_perm[i] = acc;
  if (y) {
    const int tgt = scatter ? scatter[r] : r;
    unsafeAtomicAdd(y + (size_t)tgt * d + c, (row_w ? row_w[r] : 1.f) * acc);
  }
}

int max_tiles_m(int rows, int E) {
  // sum_e ceil(c_e / BM) <= floor((rows + E (BM - 1)) / BM)
  return (int)(((long long)rows + (long long)E * (BM - 1)) / BM);
}

}  // namespace

size_t ffn_workspace_bytes(int E, int rows, int d, int f) {
  (void)E; (void)rows; (void)d; (void)f;
  return 0;
}

hipError_t launch_expert_up(const void* x, const int32_t* gather_idx, const int32_t* offsets,
                            int E, int rows, int d, int f, bool bf16, const void* W_gate,
                            const void* W_up, void* a_out, void* ws, hipStream_t s) {
  (void)ws;
  if (rows == 0) return hipSuccess;
  if (!bf16) {
    const size_t n = (size_t)rows * f;
    hipLaunchKernelGGL(up_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(x), gather_idx, offsets, E, rows, d, f,
                       static_cast<const float*>(W_gate), static_cast<const float*>(W_up),
                       static_cast<float*>(a_out));
    return hipGetLastError();
  }
  GemmArgs p{};
  p.A = static_cast<const bf16_t*>(x);
  p.gather = gather_idx;
  p.offsets = offsets;
  p.E = E; p.rows = rows; p.K = d; p.N = f;
  p.B0 = static_cast<const bf16_t*>(W_gate);
  p.B1 = static_cast<const bf16_t*>(W_up);
  p.a_out = static_cast<bf16_t*>(a_out);
  p.tiles_n = cdiv(f, BNA / 2);
  const long long tiles = (long long)max_tiles_m(rows, E) * p.tiles_n;
  const long long grid = (tiles + 7) / 8 * 8;
  p.grid_per_xcd = (int)(grid / 8);
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_expert_down(const void* a, const int32_t* offsets, int E, int rows, int f,
                              int d, bool bf16, const void* W_down, float* y_perm,
                              const int32_t* scatter_idx, const float* row_w, float* y, void* ws,
                              hipStream_t s) {
  (void)ws;
  if (rows == 0) return hipSuccess;
  if (!bf16) {
    const size_t n = (size_t)rows * d;
    hipLaunchKernelGGL(down_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(a), offsets, E, rows, f, d,
                       static_cast<const float*>(W_down), y_perm, scatter_idx, row_w, y);
    return hipGetLastError();
  }
  GemmArgs p{};
  p.A = static_cast<const bf16_t*>(a);
  p.gather = nullptr;
  p.offsets = offsets;
  p.E = E; p.rows = rows; p.K = f; p.N = d;
  p.B0 = static_cast<const bf16_t*>(W_down);
  p.B1 = nullptr;
  p.y_perm = y_perm;
  p.scatter = scatter_idx;
  p.row_w = row_w;
  p.y = y;
  p.tiles_n = cdiv(d, BNA);
  const long long tiles = (long long)max_tiles_m(rows, E) * p.tiles_n;
  const long long grid = (tiles + 7) / 8 * 8;
  p.grid_per_xcd = (int)(grid / 8);
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
