// Backward grouped GEMMs of the expert FFN (bf16 operands, fp32 accumulation).
//
// The gradients of the two expert GEMMs ("layer 0" and "layer 1", COMET
// page, "COMET's Technical Principles") for training, which the pages are
// about (COMET page, "What Is COMET"; DisagMoE page, "2.2 AF-Pipe", backward
// stream):
//
//   data gradient (DGRAD), grouped by the permuted rows of each expert:
//     C[r, n] = sum_k A[r, k] B_e[n, k]          A [rows, K], B_e [N, K]
//     layer 1: dA = dY W_down[e]^T (N = f, K = d), epilogue = SwiGLU backward
//              (dH = dA u SiLU'(h), dU = dA SiLU(h), written as [rows, 2f] bf16);
//     layer 0: dX = dH W_gate[e]^T + dU W_up[e]^T (N = d, K = 2f: the K range is
//              W_gate's rows then W_up's), epilogue = fp32 store (or add);
//   weight gradient (WGRAD), one K range per expert (its permuted rows):
//     C_e[m, n] = sum_{r in e} A[g(r), m] B[r, n]
//     layer 1: dW_down[e] = act^T dY (M = f, N = d);
//     layer 0: [dW_gate[e] | dW_up[e]] = x_perm^T [dH | dU] (M = d, N = 2f,
//              rows of x gathered through the permutation).
//
// Kernel: 4 wave64s (2 x 2) per 128 x 128 tile, each wave 64 x 64 = 4 x 4
// blocks of v_mfma_f32_16x16x32_bf16; K stages of 32; operands move HBM ->
// LDS with direct-to-LDS loads (global_load_lds_dwordx4, no register
// staging) into a ring of 4 stages, issued 3 stages ahead; one barrier per
// stage.
//   K-contiguous operands (DGRAD): LDS [128 rows][32 K], the 16-byte chunk
//     index XOR-ed with (row / 4) % 4 so that a fragment read (16 rows at one
//     chunk per 16 lanes) touches every bank once; read with ds_read_b128.
//   K-outer operands (WGRAD): LDS [32 K rows][128 columns], 32-byte pairs
//     swizzled by the K row, read with ds_read_b64_tr_b16 (the gfx950 LDS
//     transpose read: each lane receives 4 consecutive K values of one column).
// Out-of-range rows, columns and K are loaded as zeros and never stored.
// Every sum runs in a fixed order: the results are deterministic.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int NT = 256;                  // 4 waves
constexpr int OP_BYTES = BM * BK * 2;    // one operand stage: 8 KiB (both layouts)
constexpr int STAGE = 2 * OP_BYTES;      // A then B

enum { DGRAD = 0, WGRAD = 1 };
enum { EPI_SWIGLU_BWD = 0, EPI_F32 = 1, EPI_WGRAD = 2 };

struct BwdArgs {
  const bf16_t* A;          // DGRAD: [rows, K], K contiguous; WGRAD: [*, M], M contiguous
  int lda;                  // row stride of A in elements
  const int32_t* a_gather;  // WGRAD: row r of the K range reads A row a_gather[r] (or r)
  const bf16_t* B0;         // DGRAD: [E, N, K0] (K contiguous); WGRAD: [rows, N]
  const bf16_t* B1;         // DGRAD: [E, N, K1] for k >= K0, or NULL
  int K0, K1;               // DGRAD: K = K0 + K1
  int ldb;                  // WGRAD: row stride of B
  const int32_t* offsets;   // [E+1]
  int E, M, N, K;           // DGRAD: M = rows, K = K0 + K1; WGRAD: M, N (K from offsets)
  int tiles_n, tiles_m;
  // EPI_SWIGLU_BWD: h, u [rows, N] bf16 in, dhu [rows, 2N] bf16 out
  const bf16_t* h;
  const bf16_t* u;
  bf16_t* dhu;
  // EPI_F32: out [rows, N] fp32 (added to when accumulate)
  float* out;
  int accumulate;
  // EPI_WGRAD: columns n < n_split go to w0 [E, M, n_split], the rest to w1 [E, M, N - n_split]
  float* w0;
  float* w1;
  int n_split;
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ int kc_off(int row, int chunk) {
  return row * (BK * 2) + ((chunk ^ ((row >> 2) & 3)) << 4);
}
__device__ __forceinline__ int ko_swz(int krow) { return (((krow & 7) << 1) + (krow & 8)) & 15; }
__device__ __forceinline__ int ko_off(int krow, int col) {
  return krow * (BN * 2) + (((col >> 3) ^ ko_swz(krow)) << 4) + ((col & 7) << 1);
}

// (expert, m-tile, n-tile) of DGRAD tile `tile` from the device offsets: M
// tiles of an expert = ceil(c_e / BM); walk M fastest inside an (expert, N
// panel).  Every wave computes the same answer (4 experts per lane).
struct Loc {
  int e, row0, row_end, n_t;
  bool ok;
};
__device__ __forceinline__ Loc locate_dgrad(const BwdArgs& p, int tile) {
  const int lane = threadIdx.x & 63;
  int cnt[4], mt[4], off[4];
  int lane_sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    int m = 0, o = 0;
    if (e < p.E) {
      o = p.offsets[e];
      m = cdiv(p.offsets[e + 1] - o, BM);
    }
    mt[q] = m;
    off[q] = o;
    cnt[q] = m * p.tiles_n;
    lane_sum += cnt[q];
  }
  int incl = lane_sum;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int v = __shfl_up(incl, s);
    if (lane >= s) incl += v;
  }
  int start = incl - lane_sum;
  int he = -1, hs = 0, hm = 0, ho = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (tile >= start && tile < start + cnt[q]) {
      he = lane * 4 + q;
      hs = start;
      hm = mt[q];
      ho = off[q];
    }
    start += cnt[q];
  }
  const uint64_t hit = __ballot(he >= 0);
  Loc L{};
  L.ok = hit != 0;
  if (!L.ok) return L;
  const int src = __ffsll((unsigned long long)hit) - 1;
  L.e = __shfl(he, src);
  const int local = tile - __shfl(hs, src);
  const int tmt = __shfl(hm, src);
  L.n_t = local / tmt;
  const int m_t = local - L.n_t * tmt;
  L.row0 = __shfl(ho, src) + m_t * BM;
  L.row_end = min(L.row0 + BM, p.offsets[L.e + 1]);
  return L;
}

// 16 zero bytes: chunks outside the operand (rows, columns or K past the
// end) are loaded from here, so they arrive in LDS as zeros
__device__ __attribute__((aligned(16))) const bf16_t kZeroBwd[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// One direct-to-LDS load: 64 lanes x 16 bytes from their global addresses to
// the 1 KiB of LDS at lds_addr (wave-uniform).  Inline assembly, so the
// compiler's wait-count pass does not model it: the ring's waits are explicit
// (wait_loads) and ordering against the LDS reads comes from s_barrier.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "s"(lds_addr)
      : "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

constexpr int NS = 4;              // LDS ring: stages in flight
constexpr int LPW = 4;             // loads per wave per stage (2 of A, 2 of B)

// wait until at most `later` stages of this wave's loads are outstanding
__device__ __forceinline__ void wait_loads(int later) {
  if (later >= 2) wait_vm<2 * LPW>();
  else if (later == 1) wait_vm<LPW>();
  else wait_vm<0>();
}

template <int MODE, int EPI>
__global__ __launch_bounds__(NT) void grouped_gemm_bwd_kernel(BwdArgs p) {
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds;

  // ---- the tile
  int e, m0, n0, row_end = 0, k_beg = 0, nk;
  if (MODE == DGRAD) {
    const Loc L = locate_dgrad(p, blockIdx.x);
    if (!L.ok) return;
    e = __builtin_amdgcn_readfirstlane(L.e);
    m0 = __builtin_amdgcn_readfirstlane(L.row0);
    row_end = __builtin_amdgcn_readfirstlane(L.row_end);
    n0 = __builtin_amdgcn_readfirstlane(L.n_t) * BN;
    nk = cdiv(p.K, BK);
  } else {
    const int per_e = p.tiles_m * p.tiles_n;
    e = blockIdx.x / per_e;
    const int local = blockIdx.x - e * per_e;
    const int n_t = local / p.tiles_m;
    m0 = (local - n_t * p.tiles_m) * BM;
    n0 = n_t * BN;
    k_beg = __builtin_amdgcn_readfirstlane(p.offsets[e]);
    row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);  // end of the K range
    nk = cdiv(row_end - k_beg, BK);
  }

  // ---- this wave's loads: A and B loads j = 2 wave + q (q = 0, 1), each
  // filling 1 KiB of its operand's stage.  K-contiguous: rows 16 j .. 16 j + 15
  // x 4 chunks; K-outer: K rows 4 j .. 4 j + 3 x 16 chunks.  The LDS swizzle
  // is applied on the global side: lane i fills physical chunk i of the 1 KiB
  // and reads the logical chunk that belongs there.
  int a_row[2], a_col[2], b_row[2], b_col[2];  // per load: row / column of the lane's chunk
  const bf16_t* a_ptr[2];                       // DGRAD: the lane's A row
  const bf16_t* b0_ptr[2];                      // DGRAD: the lane's B0 / B1 rows
  const bf16_t* b1_ptr[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = 2 * wave + q;
    if (MODE == DGRAD) {
      const int row = 16 * j + (lane >> 2);
      const int lc = (lane & 3) ^ ((row >> 2) & 3);
      const int r = m0 + row, n = n0 + row;
      a_col[q] = b_col[q] = lc * 8;           // K offset inside the stage
      a_row[q] = r < row_end ? r : -1;
      b_row[q] = n < p.N ? n : -1;
      a_ptr[q] = p.A + (size_t)(r < row_end ? r : 0) * p.lda;
      const size_t bn = (size_t)e * p.N + (n < p.N ? n : 0);
      b0_ptr[q] = p.B0 + bn * p.K0;
      b1_ptr[q] = p.B1 ? p.B1 + bn * p.K1 - p.K0 : nullptr;  // indexed by k >= K0
    } else {
      const int krow = 4 * j + (lane >> 4);
      const int lc = (lane & 15) ^ ko_swz(krow);
      a_row[q] = b_row[q] = krow;             // K row inside the stage
      a_col[q] = m0 + lc * 8;
      b_col[q] = n0 + lc * 8;
      a_ptr[q] = b0_ptr[q] = b1_ptr[q] = nullptr;
    }
  }

  // WGRAD with a row gather: this wave's 8 K rows of a stage (8 wave .. 8
  // wave + 7) read A rows a_gather[r].  The indices are fetched with scalar
  // loads (a uniform address through the constant address space) one stage
  // before they are needed, so the vector-memory counter the ring waits on
  // counts only the ring's own loads.
  typedef __attribute__((address_space(4))) const int32_t* cidx_t;
  const cidx_t gidx = (cidx_t)p.a_gather;
  const bool gather = MODE == WGRAD && p.a_gather != nullptr;
  int gi[8];
  auto fetch_gather = [&](int st) {
    const int base = k_beg + st * BK + 8 * wave, last = row_end - 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) gi[i] = gidx[min(base + i, last)];
  };

  auto issue_stage = [&](int s) {
    const uint32_t base = lds0 + (uint32_t)((s % NS) * STAGE);
    const int kk = s * BK;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = 2 * wave + q;
      const void* ga = kZeroBwd;
      const void* gb = kZeroBwd;
      if (MODE == DGRAD) {
        const int k = kk + a_col[q];
        if (a_row[q] >= 0 && k < p.K) ga = a_ptr[q] + k;
        if (b_row[q] >= 0 && k < p.K) gb = k < p.K0 ? b0_ptr[q] + k : b1_ptr[q] + k;
      } else {
        const int r = k_beg + kk + a_row[q];
        if (r < row_end) {
          if (a_col[q] < p.M) {
            int src = r;
            if (gather) {
              const int g = lane >> 4;  // K row 8 wave + 4 q + g
              const int lo = g & 1 ? gi[4 * q + 1] : gi[4 * q];
              const int hi = g & 1 ? gi[4 * q + 3] : gi[4 * q + 2];
              src = g & 2 ? hi : lo;
            }
            ga = p.A + (size_t)src * p.lda + a_col[q];
          }
          if (b_col[q] < p.N) gb = p.B0 + (size_t)r * p.ldb + b_col[q];
        }
      }
      dma16(ga, base + (uint32_t)(j * 1024));
      dma16(gb, base + (uint32_t)(OP_BYTES + j * 1024));
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment read offsets (bytes inside an operand stage)
  int fa_off[4], fb_off[4], fa_off4[4], fb_off4[4];
  {
    const int l15 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (MODE == DGRAD) {
        fa_off[i] = kc_off(wm * 64 + i * 16 + l15, g);
        fb_off[i] = kc_off(wn * 64 + i * 16 + l15, g);
        fa_off4[i] = fb_off4[i] = 0;
      } else {
        const int kr = g * 8 + (l15 >> 2);
        const int ca = wm * 64 + i * 16 + (lane & 3) * 4;
        const int cb = wn * 64 + i * 16 + (lane & 3) * 4;
        fa_off[i] = ko_off(kr, ca);
        fa_off4[i] = ko_off(kr + 4, ca);
        fb_off[i] = ko_off(kr, cb);
        fb_off4[i] = ko_off(kr + 4, cb);
      }
    }
  }

  // prologue: stages 0 .. NS - 2
  for (int s0 = 0; s0 < NS - 1 && s0 < nk; ++s0) {
    if (gather) fetch_gather(s0);
    issue_stage(s0);
  }
  if (gather && NS - 1 < nk) fetch_gather(NS - 1);
  for (int s = 0; s < nk; ++s) {
    // stage s has landed once only stages s + 1 .. s + NS - 2 (if they exist)
    // remain; the barrier makes every wave's loads of stage s visible and
    // ends every wave's reads of slot (s - 1) % NS, which stage s + NS - 1 refills
    wait_loads(min(NS - 2, nk - 1 - s));
    __syncthreads();
    if (s + NS - 1 < nk) {
      issue_stage(s + NS - 1);
      if (gather && s + NS < nk) fetch_gather(s + NS);
    }
    const char* As = lds + (s % NS) * STAGE;
    const char* Bs = As + OP_BYTES;
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (MODE == DGRAD) {
        fa[i] = *reinterpret_cast<const bf16x8*>(As + fa_off[i]);
        fb[i] = *reinterpret_cast<const bf16x8*>(Bs + fb_off[i]);
      } else {
        const bf16x4 alo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(As + fa_off[i]));
        const bf16x4 ahi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(As + fa_off4[i]));
        fa[i] = __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x4 blo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Bs + fb_off[i]));
        const bf16x4 bhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Bs + fb_off4[i]));
        fb[i] = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }

  // ---- epilogue (accumulator layout: column lane % 16, rows 4 (lane / 16) + q)
  const int col_l = lane & 15, row_l = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * 64 + i * 16 + row_l + q;
        const int n = n0 + wn * 64 + j * 16 + col_l;
        const float v = acc[i][j][q];
        if (MODE == DGRAD) {
          if (m >= row_end || n >= p.N) continue;
          if (EPI == EPI_SWIGLU_BWD) {
            const size_t hi = (size_t)m * p.N + n;
            const float h = bf16_to_f32(p.h[hi]), u = bf16_to_f32(p.u[hi]);
            const float sg = 1.f / (1.f + __expf(-h));
            const float dh = v * u * sg * (1.f + h * (1.f - sg));
            const float du = v * h * sg;
            p.dhu[(size_t)m * 2 * p.N + n] = f32_to_bf16(dh);
            p.dhu[(size_t)m * 2 * p.N + p.N + n] = f32_to_bf16(du);
          } else {
            float* o = p.out + (size_t)m * p.N + n;
            *o = p.accumulate ? *o + v : v;
          }
        } else {
          if (m >= p.M || n >= p.N) continue;
          if (n < p.n_split)
            p.w0[((size_t)e * p.M + m) * p.n_split + n] = v;
          else
            p.w1[((size_t)e * p.M + m) * (p.N - p.n_split) + (n - p.n_split)] = v;
        }
      }
}

int dgrad_grid(int rows, int E, int tiles_n) {
  // sum_e ceil(c_e / BM) <= floor((rows + E (BM - 1)) / BM)
  const long long mt = ((long long)rows + (long long)E * (BM - 1)) / BM;
  return (int)(mt * tiles_n);
}

}  // namespace

hipError_t launch_expert_down_backward(const void* dy_perm, const int32_t* offsets, int E,
                                       int rows, int f, int d, const void* W_down,
                                       const void* h, const void* u, const void* act,
                                       void* dhu, float* dW_down, hipStream_t s) {
  if (rows > 0) {
    // dA = dY W_down[e]^T with the SwiGLU backward in the epilogue
    BwdArgs p{};
    p.A = static_cast<const bf16_t*>(dy_perm);
    p.lda = d;
    p.B0 = static_cast<const bf16_t*>(W_down);  // [E, f, d]: row n of expert e has d contiguous
    p.K0 = d;
    p.K1 = 0;
    p.offsets = offsets;
    p.E = E;
    p.M = rows;
    p.N = f;
    p.K = d;
    p.tiles_n = cdiv(f, BN);
    p.h = static_cast<const bf16_t*>(h);
    p.u = static_cast<const bf16_t*>(u);
    p.dhu = static_cast<bf16_t*>(dhu);
    const int grid = dgrad_grid(rows, E, p.tiles_n);
    if (grid > 0)
      hipLaunchKernelGGL((grouped_gemm_bwd_kernel<DGRAD, EPI_SWIGLU_BWD>), dim3(grid), dim3(NT), 0,
                         s, p);
  }
  // dW_down[e] = act_e^T dY_e (every expert, empty ones get zeros)
  BwdArgs q{};
  q.A = static_cast<const bf16_t*>(act);
  q.lda = f;
  q.B0 = static_cast<const bf16_t*>(dy_perm);
  q.ldb = d;
  q.offsets = offsets;
  q.E = E;
  q.M = f;
  q.N = d;
  q.tiles_m = cdiv(f, BM);
  q.tiles_n = cdiv(d, BN);
  q.w0 = dW_down;
  q.n_split = d;
  hipLaunchKernelGGL((grouped_gemm_bwd_kernel<WGRAD, EPI_WGRAD>),
                     dim3((unsigned)(E * q.tiles_m * q.tiles_n)), dim3(NT), 0, s, q);
  return hipGetLastError();
}

hipError_t launch_expert_up_backward(const void* x, const int32_t* gather_idx,
                                     const int32_t* offsets, int E, int rows, int d, int f,
                                     const void* W_gate, const void* W_up, const void* dhu,
                                     float* dx_perm, int accumulate, float* dW_gate,
                                     float* dW_up, hipStream_t s) {
  if (rows > 0) {
    // dX = dH W_gate[e]^T + dU W_up[e]^T: K runs over W_gate's f columns, then W_up's
    BwdArgs p{};
    p.A = static_cast<const bf16_t*>(dhu);
    p.lda = 2 * f;
    p.B0 = static_cast<const bf16_t*>(W_gate);  // [E, d, f]: row n of expert e has f contiguous
    p.B1 = static_cast<const bf16_t*>(W_up);
    p.K0 = f;
    p.K1 = f;
    p.offsets = offsets;
    p.E = E;
    p.M = rows;
    p.N = d;
    p.K = 2 * f;
    p.tiles_n = cdiv(d, BN);
    p.out = dx_perm;
    p.accumulate = accumulate;
    const int grid = dgrad_grid(rows, E, p.tiles_n);
    if (grid > 0)
      hipLaunchKernelGGL((grouped_gemm_bwd_kernel<DGRAD, EPI_F32>), dim3(grid), dim3(NT), 0, s, p);
  }
  // [dW_gate[e] | dW_up[e]] = x_perm_e^T [dH_e | dU_e]
  BwdArgs q{};
  q.A = static_cast<const bf16_t*>(x);
  q.lda = d;
  q.a_gather = gather_idx;
  q.B0 = static_cast<const bf16_t*>(dhu);
  q.ldb = 2 * f;
  q.offsets = offsets;
  q.E = E;
  q.M = d;
  q.N = 2 * f;
  q.tiles_m = cdiv(d, BM);
  q.tiles_n = cdiv(2 * f, BN);
  q.w0 = dW_gate;
  q.w1 = dW_up;
  q.n_split = f;
  hipLaunchKernelGGL((grouped_gemm_bwd_kernel<WGRAD, EPI_WGRAD>),
                     dim3((unsigned)(E * q.tiles_m * q.tiles_n)), dim3(NT), 0, s, q);
  return hipGetLastError();
}

}  // namespace moe
