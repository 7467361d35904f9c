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
// Kernels:
//   * grouped_gemm_bwd256_kernel (and the _pair form that runs a layer's
//     DGRAD and WGRAD tiles in one launch): the forward's ping-pong design,
//     256 x 256 tiles, 8 waves in two groups taking turns between fragment
//     reads + loads and 64 MFMAs per K stage of 64, A ring 2 / B ring 3 in
//     160 KiB of LDS, direct-to-LDS loads (global_load_lds_dwordx4) with the
//     swizzle applied on the global side, epilogues staged through LDS so
//     every global access is 16 bytes per lane;
//   * grouped_gemm_bwd_kernel: 4 wave64s (2 x 2) per 128 x 128 tile, K stages
//     of 32 in a ring of 4; it serves the layer-0 weight gradient when the
//     rows of x are gathered through the permutation.
// LDS layouts:
//   K-contiguous operands (DGRAD): [rows][K], the 16-byte chunk index XOR-ed
//     by the row so that a fragment read touches every bank once; read with
//     ds_read_b128.
//   K-outer operands (WGRAD): [K rows][columns], 32-byte pairs swizzled by
//     the K row, read with ds_read_b64_tr_b16 (the gfx950 LDS transpose read:
//     each lane receives 4 consecutive K values of one column).
// Rows and columns past an operand read zeros or a valid row, and their
// results are never stored; K past the operand is zero-filled.
// Every sum runs in a fixed order: the results are deterministic.
#include "moe_internal.h"

#include <algorithm>

namespace moe {
// compute units of the current device (cached per device; 256 if unknown)
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int NT = 256;                  // 4 waves
constexpr int OP_BYTES = BM * BK * 2;    // one operand stage: 8 KiB (both layouts)
constexpr int STAGE = 2 * OP_BYTES;      // A then B

enum { DGRAD = 0, WGRAD = 1 };
// EPI_F32_ADD: EPI_F32 adding to out (accumulate = 1), a variant of its own so
// that the common, store-only epilogue carries none of the loads' waits
enum { EPI_SWIGLU_BWD = 0, EPI_F32 = 1, EPI_WGRAD = 2, EPI_F32_ADD = 3 };

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
  // WGRAD K split: each expert's rows are cut in ksplit chunks; chunk c of
  // expert e writes its partial C_e as slab e * ksplit + c of w0 (the host
  // points w0 at the workspace, n_split = N) and wgrad_sum_kernel adds the
  // chunks in order into the weight gradients (ksplit = 1: straight to w0 / w1)
  int ksplit;
  float* part;  // host side only: the workspace, before w0 is pointed at it
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
  const int incl = wave_incl_sum(lane_sum);
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
  const int src = __ffsll((unsigned long long)hit) - 1;  // uniform: read from that lane
  L.e = __builtin_amdgcn_readlane(he, src);
  const int local = tile - __builtin_amdgcn_readlane(hs, src);
  const int tmt = __builtin_amdgcn_readlane(hm, src);
  L.n_t = local / tmt;
  const int m_t = local - L.n_t * tmt;
  L.row0 = __builtin_amdgcn_readlane(ho, src) + m_t * BM;
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

// ------------------------------------------------------------------------
// 256 x 256 tiles in ping-pong (the large-tile kernel).  8 waves in two
// groups of 4: group X computes the tile's first 128 rows and issues the A
// loads, group Y the last 128 rows and issues the B loads; each wave owns
// 128 x 64 (8 x 4 blocks of 16 x 16).  The groups alternate between a
// memory phase (fragment reads from LDS and the next stage's loads) and a
// compute phase (64 MFMAs per K stage of 64), so one group's MFMAs overlap
// the other's LDS traffic on every SIMD; MFMAs run at raised wave priority.
// Against the 128 x 128 tile, a wave issues 4 MFMAs per 16-byte fragment
// read instead of 2.  LDS: A ring of 2 stages, B ring of 3 (160 KiB).
// ------------------------------------------------------------------------
namespace bpp {
constexpr int PBK = 64, RA = 2, RB = 3, MI = 8, NJ = 4, KS = PBK / 32, LD = 8;
constexpr int SLOT = 256 * PBK * 2;          // one operand stage: 32 KiB
constexpr int HALF = PBK * 128 * 2;          // K-outer: one 128-column half of a stage
constexpr int B_RING = RA * SLOT;            // B slots follow the A slots
constexpr int LDS_BYTES = (RA + RB) * SLOT;  // 160 KiB
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

// K-contiguous stage [256 rows][64 K]: 16-byte chunk index XOR-ed with
// (row / 2) % 8 (a fragment read, 16 rows at one chunk, touches every bank
// once); K-outer stage: two halves [64 K rows][128 columns] with the 32-byte
// pair swizzle of the 128 x 128 kernel above.
__device__ __forceinline__ lds_bf16x4* lds_at(uint32_t a) { return (lds_bf16x4*)(uintptr_t)a; }
__device__ __forceinline__ int kc2_off(int row, int chunk) {
  return row * (PBK * 2) + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <int N>
__device__ __forceinline__ void wait_groups(int n) {
  if (n >= 2) wait_vm<2 * N>();
  else if (n == 1) wait_vm<N>();
  else wait_vm<0>();
}

// The DGRAD tile: (expert, 256-row M tile, N panel), M fastest inside an
// (expert, N panel).  An expert's c rows form ceil(c / 16) blocks of 16
// dealt evenly to its ceil(c / 256) M tiles (the first ones take one more),
// so the tiles sharing a panel take equal time and only the expert's last
// block is padded.
struct PTile {
  int e, row0, row_end, nb, n_t;
  bool ok;
};
__device__ __forceinline__ PTile locate_dgrad256(const BwdArgs& p, int tile) {
  const int lane = threadIdx.x & 63;
  int cnt[4], mt[4], off[4];
  int lane_sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    int m = 0, o = 0;
    if (e < p.E) {
      o = p.offsets[e];
      m = cdiv(p.offsets[e + 1] - o, 256);
    }
    mt[q] = m;
    off[q] = o;
    cnt[q] = m * p.tiles_n;
    lane_sum += cnt[q];
  }
  const int incl = wave_incl_sum(lane_sum);
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
  PTile L{};
  L.ok = hit != 0;
  if (!L.ok) return L;
  const int src = __ffsll((unsigned long long)hit) - 1;  // uniform: read from that lane
  L.e = __builtin_amdgcn_readlane(he, src);
  const int local = tile - __builtin_amdgcn_readlane(hs, src);
  const int tmt = __builtin_amdgcn_readlane(hm, src);
  const int toff = __builtin_amdgcn_readlane(ho, src);
  L.n_t = local / tmt;
  const int m_t = local - L.n_t * tmt;
  const int c_e = p.offsets[L.e + 1] - toff;
  const int nbe = cdiv(c_e, 16);
  const int b_lo = nbe / tmt, b_rem = nbe - b_lo * tmt;
  const int b0 = m_t * b_lo + min(m_t, b_rem);
  const int b1 = b0 + b_lo + (m_t < b_rem ? 1 : 0);
  L.nb = b1 - b0;
  L.row0 = toff + 16 * b0;
  L.row_end = min(toff + 16 * b1, toff + c_e);
  return L;
}
}  // namespace bpp

// One direct-to-LDS load with a scalar base: lane i reads 16 bytes at
// base + voff_i and writes LDS bytes lds_addr + 16 i.
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* base, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "m0");
}

__device__ __forceinline__ const char* uniform_ptr(const void* q) {
  const uint64_t v = (uint64_t)(uintptr_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// FASTK (DGRAD with K and K0 multiples of 64): no stage straddles the end of
// K or the W_gate / W_up boundary, so every load of a stage shares one scalar
// base and each lane keeps one 32-bit byte offset per load (rows past the
// operand read the tile's first row; their results are never stored).
// The body of one workgroup: block `bid` of a launch of G blocks, LDS at
// `lds` (LDS_BYTES, 1 KiB aligned).
template <int MODE, int EPI, bool FASTK>
__device__ __forceinline__ void bwd256_body(const BwdArgs& p, char* lds, const int bid,
                                            const int G) {
  using namespace bpp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool X = wave < 4;  // X: tile rows 0-127, issues the A loads; Y: rows 128-255, B loads
  const int wg = wave & 3;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds;

  // ---- the tile.  DGRAD tiles cost the same (K is fixed): XCD-aware, the
  // grid a multiple of 8 and consecutive tiles, which share a weight panel,
  // on the same XCD's L2.  WGRAD tiles cost their expert's rows: dealt
  // round-robin (block order), so every XCD gets a share of every expert.
  const int tile = MODE == DGRAD ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
  int e, n0, m0 = 0, row0 = 0, row_end = 0, k_beg = 0, nk, my_nb, grow0, nb = 8, nbx = 4;
  int kchunk = 0;  // WGRAD: the K chunk of a split expert
  if (MODE == DGRAD) {
    const PTile L = locate_dgrad256(p, tile);
    if (!L.ok) return;
    e = __builtin_amdgcn_readfirstlane(L.e);
    row0 = __builtin_amdgcn_readfirstlane(L.row0);
    row_end = __builtin_amdgcn_readfirstlane(L.row_end);
    n0 = __builtin_amdgcn_readfirstlane(L.n_t) * 256;
    nb = __builtin_amdgcn_readfirstlane(L.nb);
    nbx = (nb + 1) >> 1;              // X takes the first ceil(nb / 2) blocks, Y the rest
    my_nb = X ? nbx : nb - nbx;
    grow0 = X ? 0 : 16 * nbx;
    nk = cdiv(p.K, PBK);
  } else {
    const int per_c = p.tiles_m * p.tiles_n;
    const int per_e = per_c * p.ksplit;
    e = tile / per_e;
    if (e >= p.E) return;
    const int lc = tile - e * per_e;
    kchunk = lc / per_c;
    const int local = lc - kchunk * per_c;
    // the side with fewer panels runs fastest, so the tiles running side by
    // side read the operand with more panels once
    int m_t, n_t;
    if (p.tiles_n <= p.tiles_m) {
      m_t = local / p.tiles_n;
      n_t = local - m_t * p.tiles_n;
    } else {
      n_t = local / p.tiles_m;
      m_t = local - n_t * p.tiles_m;
    }
    m0 = m_t * 256;
    n0 = n_t * 256;
    grow0 = X ? 0 : 128;
    my_nb = min(MI, max(0, cdiv(p.M - (m0 + grow0), 16)));
    k_beg = __builtin_amdgcn_readfirstlane(p.offsets[e]);
    row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
    if (p.ksplit > 1) {  // chunk kchunk of the expert's rows (stages of PBK; may be empty)
      const int kc = cdiv(cdiv(row_end - k_beg, p.ksplit), PBK) * PBK;
      k_beg = min(row_end, k_beg + kchunk * kc);
      row_end = min(row_end, k_beg + kc);
      e = e * p.ksplit + kchunk;  // output slab of the partial (w0 = part, n_split = N)
    }
    nk = cdiv(row_end - k_beg, PBK);
  }

  // ---- this wave's 8 loads per stage (1 KiB each), q = 0..7
  //   K-contiguous (DGRAD): LDS rows 64 wg + 8 q + lane / 8, chunk lane % 8;
  //     A: LDS rows 0-127 are group X's blocks, 128-255 group Y's; B: LDS row
  //     = column n0 + row of the output;
  //   K-outer (WGRAD): half wg / 2, K rows 32 (wg % 2) + 4 q + lane / 16,
  //     chunk lane % 16 (A half = 128 M columns, B half = 128 N columns).
  // The swizzle is applied on the global side: lane i fills physical chunk
  // i.  DGRAD: load q of a wave covers operand rows rb + 8 q + lane / 8
  // (rb: the wave's first row; those with lane / 8 + 8 q < ld_lim exist),
  // at element offset ld_lane + q ld_step from the tile's base.  Addresses
  // are formed at issue.
  const bf16_t* base0 = p.A;
  const bf16_t* base1 = p.A;
  int k_split = p.K;  // k < k_split reads base0, the rest base1
  int ld_lane = 0, ld_lim = 0, ld_step = 0;
  int ko_col = 0;  // WGRAD: the wave's first column
  if (MODE == DGRAD) {
    int rb, stride;
    if (X) {
      // LDS rows 0-127 (waves 0, 1): group X's blocks; 128-255: group Y's
      base0 = base1 = p.A + (size_t)row0 * p.lda;
      const int j0 = 64 * (wg & 1);
      const int gnb = wg < 2 ? nbx : nb - nbx;
      rb = (wg < 2 ? 0 : 16 * nbx) + j0;  // row inside the tile
      ld_lim = min(16 * gnb - j0, row_end - row0 - rb);
      stride = p.lda;
    } else {
      const size_t bn = (size_t)e * p.N + n0;
      base0 = p.B0 + bn * p.K0;
      base1 = p.B1 ? p.B1 + bn * p.K0 - p.K0 : base0;  // K1 = K0; indexed by k >= K0
      k_split = p.K0;
      rb = 64 * wg;
      ld_lim = p.N - n0 - rb;
      stride = p.K0;
    }
    ld_lane = (rb + (lane >> 3)) * stride;
    ld_step = 8 * stride;
  } else {
    base0 = X ? p.A : p.B0;
    ko_col = (X ? m0 : n0) + 128 * (wg >> 1);
  }

  uint32_t fk_off[FASTK ? LD : 1];  // FASTK: byte offsets from the stage's base
  if (FASTK && MODE == DGRAD) {
#pragma unroll
    for (int q = 0; q < LD; ++q) {
      const bool ok = (lane >> 3) + 8 * q < ld_lim;
      const int kc = ((lane & 7) ^ (4 * (q & 1) + (lane >> 4))) << 3;
      fk_off[q] = (uint32_t)((ok ? ld_lane + q * ld_step : 0) + kc) * 2u;
    }
  } else if (FASTK) {
    // WGRAD: K row 32 (wg % 2) + 4 q + lane / 16 of a full stage, from the
    // stage's base row; columns past the operand read column 0 (unstored)
    const int ld = X ? p.lda : p.ldb, lim = X ? p.M : p.N;
#pragma unroll
    for (int q = 0; q < LD; ++q) {
      const int kr = 4 * q + (lane >> 4);
      int col = ko_col + (((lane & 15) ^ ko_swz(kr)) << 3);
      if (col >= lim) col = 0;
      fk_off[q] = (uint32_t)(kr * ld + col) * 2u;
    }
  }

  // issue this wave's loads of stage kt into slot `slot` of its ring
  auto issue = [&](int kt, int slot, int qa, int qb) {
    const uint32_t dst0 = lds0 + (uint32_t)((X ? 0 : B_RING) + slot * SLOT + wg * LD * 1024);
    const int kk = kt * PBK;
    if (FASTK && MODE == DGRAD) {
      const char* sb = uniform_ptr(kk < k_split ? (const void*)(base0 + kk) : (const void*)(base1 + kk));
#pragma unroll
      for (int q = qa; q < qb; ++q) dma16_s(fk_off[q], sb, dst0 + (uint32_t)(q * 1024));
      return;
    }
    if (FASTK && k_beg + kk + PBK <= row_end) {  // WGRAD, a stage of the expert's rows only
      const char* sb = uniform_ptr(base0 + (size_t)(k_beg + kk + 32 * (wg & 1)) * (X ? p.lda : p.ldb));
#pragma unroll
      for (int q = qa; q < qb; ++q) dma16_s(fk_off[q], sb, dst0 + (uint32_t)(q * 1024));
      return;
    }
#pragma unroll
    for (int q = qa; q < qb; ++q) {
      const void* ga = kZeroBwd;
      if (MODE == DGRAD) {
        // logical chunk of physical chunk lane % 8 in LDS row 64 wg + 8 q + lane / 8
        const int k = kk + (((lane & 7) ^ (4 * (q & 1) + (lane >> 4))) << 3);
        // B of layer 0 spans W_gate (k < K0) then W_up; A is one operand
        if ((lane >> 3) + 8 * q < ld_lim && k < p.K)
          ga = (k < k_split ? base0 : base1) + (ld_lane + q * ld_step) + k;
      } else {
        const int krow = 32 * (wg & 1) + 4 * q + (lane >> 4);
        const int col = ko_col + (((lane & 15) ^ ko_swz(krow)) << 3);
        const int r = k_beg + kk + krow;
        if (r < row_end && col < (X ? p.M : p.N))
          ga = base0 + (size_t)r * (X ? p.lda : p.ldb) + col;
      }
      dma16(ga, dst0 + (uint32_t)(q * 1024));
    }
  };

  // ---- fragment read offsets (bytes inside a stage slot).  K step 1 is
  // chunk + 4 (K-contiguous: the swizzle XORs it, so it has its own
  // offset) or 32 K rows further (K-outer: + 8 KiB).  Blocks: K-contiguous
  // + 16 rows = + 2 KiB; K-outer + 16 columns = the offset XOR 32 bytes
  // (the swizzle XORs into the same bits).
  const int l15 = lane & 15, g = lane >> 4;
  int fa_off[2], fb_off[2];
  if (MODE == DGRAD) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fa_off[ks] = kc2_off((X ? 0 : 128) + l15, ks * 4 + g);
      fb_off[ks] = kc2_off(wg * 64 + l15, ks * 4 + g);
    }
  } else {
    const int kr = g * 8 + (l15 >> 2), c = (lane & 3) * 4;
    // [0]: K rows kr, [1]: kr + 4 (the two halves of a transposed read)
    fa_off[0] = (X ? 0 : HALF) + ko_off(kr, c);
    fa_off[1] = (X ? 0 : HALF) + ko_off(kr + 4, c);
    fb_off[0] = (wg >> 1) * HALF + ko_off(kr, (wg & 1) * 64 + c);
    fb_off[1] = (wg >> 1) * HALF + ko_off(kr + 4, (wg & 1) * 64 + c);
  }

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 fa[KS][MI], fb[KS][NJ];
  // memory phase: read the stage's fragments (A slot sa, B slot sb), issue
  // this wave's loads of stage ld_kt into slot ld_slot (the slot of the stage
  // before, which no wave reads any more), wait for the reads.  The scalar-
  // base form issues half its loads after each K step's reads (+0.8%); the
  // per-lane form issues first, which keeps its 64-bit load addresses and
  // the fragments from being live together (else it spills).
  auto memory = [&](int sa, int sb, int ld_kt, int ld_slot) {
    if (!FASTK && ld_kt < nk) issue(ld_kt, ld_slot, 0, LD);
    const char* As = lds + sa * SLOT;
    const char* Bs = lds + B_RING + sb * SLOT;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) {
        if (MODE == DGRAD) {
          fb[ks][nj] = *reinterpret_cast<const bf16x8*>(Bs + fb_off[ks] + nj * 16 * PBK * 2);
        } else {
          // the slot base has no bits below 1 KiB: XOR-ing the sum equals
          // XOR-ing the offset, and keeps the per-block addresses inside the
          // loop (transient) instead of 24 hoisted registers
          const uint32_t bk = lds0 + (uint32_t)(B_RING + sb * SLOT + ks * 8192);
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_at(((bk + fb_off[0]) ^ (32 * nj))));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_at(((bk + fb_off[1]) ^ (32 * nj))));
          fb[ks][nj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (mi < my_nb) {
          if (MODE == DGRAD) {
            fa[ks][mi] = *reinterpret_cast<const bf16x8*>(As + fa_off[ks] + mi * 16 * PBK * 2);
          } else {
            const uint32_t ak = lds0 + (uint32_t)(sa * SLOT + ks * 8192);
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_at(((ak + fa_off[0]) ^ (32 * mi))));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_at(((ak + fa_off[1]) ^ (32 * mi))));
            fa[ks][mi] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
      }
      if (FASTK && ld_kt < nk) issue(ld_kt, ld_slot, ks * (LD / KS), (ks + 1) * (LD / KS));
    }
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  };
  auto compute = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (mi >= my_nb) break;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks][mi], fb[ks][nj],
                                                               acc[mi][nj], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Both groups pass the same barriers: one after the prologue, two per stage.
  if (X) {
    // prologue: A(0) .. A(RA - 2); wait for A(0)
    for (int s = 0; s < RA - 1 && s < nk; ++s) issue(s, s, 0, LD);
    wait_groups<LD>(min(RA - 2, nk - 1));
    __builtin_amdgcn_s_barrier();
    int sa = 0, sb = 0;
    for (int s = 0; s < nk; ++s) {
      const int la = sa == 0 ? RA - 1 : sa - 1;  // slot of stage s - 1 = of stage s + RA - 1
      memory(sa, sb, s + RA - 1, la);
      __builtin_amdgcn_s_barrier();
      compute();
      wait_groups<LD>(min(RA - 2, nk - 2 - s));  // A(s + 1) has landed
      __builtin_amdgcn_s_barrier();
      sa = sa == RA - 1 ? 0 : sa + 1;
      sb = sb == RB - 1 ? 0 : sb + 1;
    }
  } else {
    for (int s = 0; s < RB - 1 && s < nk; ++s) issue(s, s, 0, LD);
    wait_groups<LD>(min(RB - 2, nk - 1));
    __builtin_amdgcn_s_barrier();
    int sa = 0, sb = 0;
    for (int s = 0; s < nk; ++s) {
      if (s > 0) compute();  // stage s - 1
      __builtin_amdgcn_s_barrier();
      const int lb = sb == 0 ? RB - 1 : sb - 1;
      memory(sa, sb, s + RB - 1, lb);
      wait_groups<LD>(min(RB - 2, nk - 2 - s));  // B(s + 1) has landed
      __builtin_amdgcn_s_barrier();
      sa = sa == RA - 1 ? 0 : sa + 1;
      sb = sb == RB - 1 ? 0 : sb + 1;
    }
    if (nk > 0) compute();
  }

  // ---- epilogue.  Both groups have passed their last barrier after their
  // last LDS read, so the ring is free: each wave stages one 16-row block of
  // its 16 x 64 outputs at a time in its own LDS area (accumulator layout:
  // column lane % 16, rows 4 (lane / 16) + i) and reads it back by rows, so
  // that every global access is 16 bytes per lane.
  constexpr int SS = 64 + 4;  // staging row stride in floats
  float* st = reinterpret_cast<float*>(lds + wave * 16 * SS * 4);
  // an opaque copy of the lane index: the epilogue's lane-dependent
  // offsets cannot be hoisted above the K loop, where every register counts
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  const int col_l = lane_e & 15, row_l = (lane_e >> 4) * 4;
  const int ncol0 = n0 + wg * 64;  // the wave's first output column
  int rbase, rlim;                 // the wave's first row, its row bound
  if (MODE == DGRAD) {
    rbase = row0 + grow0;
    rlim = min(row_end, row0 + grow0 + 16 * my_nb);
  } else {
    rbase = m0 + grow0;
    rlim = p.M;
  }
  constexpr bool add = EPI == EPI_F32_ADD;
  // The epilogue's loads (h and u for the SwiGLU backward; the old dX_perm
  // when accumulating) are issued one 16-row block ahead, before the
  // previous block's stores.  vmcnt counts loads and stores together and
  // retires them in order: issued per block, every chunk's wait also drained
  // the stores before it, one memory round trip per chunk; issued ahead, the
  // wait for block mi + 1's loads leaves block mi's stores in flight and the
  // loads' latency overlaps block mi's math and stores.
  u32x4 hu[2][4];   // SwiGLU: [block parity][h, u of chunk 0, h, u of chunk 1]
  f32x4 old[2][4];  // accumulate: [block parity][chunk]
  // The loads are branch-free (a lane outside the output reads element 0,
  // in bounds whenever the tile has a row, and discards it): loads inside
  // branches make the compiler's wait counts fall back to waiting for all.
  auto prefetch = [&](int mi, int b) {
    if (EPI == EPI_SWIGLU_BWD) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int idx = c2 * 64 + lane_e, r = idx >> 3, c = (idx & 7) * 8;
        const int m = rbase + mi * 16 + r, n = ncol0 + c;
        const size_t at = m < rlim && n < p.N ? (size_t)m * p.N + n : 0;
        // h, u are read once and dH, dU are re-read only by the next
        // launch, past the last-level cache at these sizes: non-temporal
        hu[b][2 * c2] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.h + at));
        hu[b][2 * c2 + 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.u + at));
      }
    } else if (MODE == DGRAD && add) {
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int idx = c4 * 64 + lane_e, r = idx >> 4, c = (idx & 15) * 4;
        const int m = rbase + mi * 16 + r, n = ncol0 + c;
        const size_t at = m < rlim && n < p.N ? (size_t)m * p.N + n : 0;
        old[b][c4] = *reinterpret_cast<const f32x4*>(p.out + at);
      }
    }
  };
  // Every prefetch is issued, before any branch (a block past the tile's
  // rows reads element 0): a load issued on one path only would make the
  // waits after the join count as if it were not in flight, and wait for it.
  // The scheduling barriers keep the compiler from sinking the loads back to
  // their use.
  constexpr bool loads = EPI == EPI_SWIGLU_BWD || (MODE == DGRAD && add);
  if (loads) {
    prefetch(0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    if (loads) {
      if (mi + 1 < MI) prefetch(mi + 1, (mi + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // a skipped block, not an early exit: with a second exit the loop may
    // stay rolled, and acc[mi] then lives in scratch memory (3x slower)
    if (mi >= my_nb) continue;
    // the block's accumulators into the staging area
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[(row_l + i) * SS + nj * 16 + col_l] = acc[mi][nj][i];
    __builtin_amdgcn_wave_barrier();
    if (EPI == EPI_SWIGLU_BWD) {
      // 16 rows x 8 chunks of 8 columns: 2 per lane
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int idx = c2 * 64 + lane_e, r = idx >> 3, c = (idx & 7) * 8;
        const int m = rbase + mi * 16 + r, n = ncol0 + c;
        if (m < rlim && n < p.N) {
          const u32x4 hv = hu[mi & 1][2 * c2], uv = hu[mi & 1][2 * c2 + 1];
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(st + r * SS + c);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(st + r * SS + c + 4);
          u32x4 dh, du;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float dhj[2], duj[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int el = 2 * j + t;
              const float gv = el < 4 ? g0[el] : g1[el - 4];
              const float h = __uint_as_float(t ? (hv[j] & 0xffff0000u) : (hv[j] << 16));
              const float u = __uint_as_float(t ? (uv[j] & 0xffff0000u) : (uv[j] << 16));
              const float sg = 1.f / (1.f + __expf(-h));
              dhj[t] = gv * u * sg * (1.f + h * (1.f - sg));
              duj[t] = gv * h * sg;
            }
            dh[j] = pack_bf16x2(dhj[0], dhj[1]);
            du[j] = pack_bf16x2(duj[0], duj[1]);
          }
          bf16_t* d = p.dhu + (size_t)m * 2 * p.N + n;
          __builtin_nontemporal_store(dh, reinterpret_cast<u32x4*>(d));
          __builtin_nontemporal_store(du, reinterpret_cast<u32x4*>(d + p.N));
        }
      }
    } else {
      // 16 rows x 16 chunks of 4 floats: 4 per lane
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int idx = c4 * 64 + lane_e, r = idx >> 4, c = (idx & 15) * 4;
        const int m = rbase + mi * 16 + r, n = ncol0 + c;
        if (m < rlim && n < p.N) {
          f32x4 v = *reinterpret_cast<const f32x4*>(st + r * SS + c);
          float* o;
          if (MODE == DGRAD)
            o = p.out + (size_t)m * p.N + n;
          else if (n < p.n_split)
            o = p.w0 + ((size_t)e * p.M + m) * p.n_split + n;
          else
            o = p.w1 + ((size_t)e * p.M + m) * (p.N - p.n_split) + (n - p.n_split);
          if (MODE == DGRAD && add) v += old[mi & 1][c4];
          // weight gradients are not read again soon: non-temporal stores
          // keep them from evicting the operand panels of running tiles
          // from the caches (+1-2%)
          if (MODE == WGRAD)
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(o));
          else
            *reinterpret_cast<f32x4*>(o) = v;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int MODE, int EPI, bool FASTK = false>
__global__ __launch_bounds__(512, 1) void grouped_gemm_bwd256_kernel(BwdArgs p) {
  __shared__ __attribute__((aligned(1024))) char lds[bpp::LDS_BYTES];
  bwd256_body<MODE, EPI, FASTK>(p, lds, blockIdx.x, gridDim.x);
}

// Both GEMMs of one layer's backward in one launch: blocks [0, gd) are the
// data gradient's (XCD-aware over gd), the rest the weight gradient's.  The
// two are independent (they share only inputs), and blocks start in order,
// so the weight gradient's short tiles fill the compute units that the data
// gradient's last, partial round of long tiles leaves idle.
template <int EPI>
__global__ __launch_bounds__(512, 1) void grouped_gemm_bwd256_pair_kernel(BwdArgs pd, BwdArgs pw,
                                                                          int gd) {
  __shared__ __attribute__((aligned(1024))) char lds[bpp::LDS_BYTES];
  if ((int)blockIdx.x < gd)
    bwd256_body<DGRAD, EPI, true>(pd, lds, blockIdx.x, gd);
  else
    bwd256_body<WGRAD, EPI_WGRAD, true>(pw, lds, blockIdx.x - gd, gridDim.x - gd);
}

// ------------------------------------------------------------------------
// fp32 layers (small): one thread per output element, a plain FMA loop over
// K in order, as the forward's fp32 path.
// ------------------------------------------------------------------------
__device__ __forceinline__ int expert_of_row_b(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E;  // e with offsets[e] <= r < offsets[e + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// dA[r, n] = sum_k dY[r, k] W_down[e][n, k]; dhu[r, n] = dA u s (1 + h (1 - s)),
// dhu[r, f + n] = dA h s, s = sigmoid(h)
__global__ void down_bwd_dgrad_f32_kernel(const float* __restrict__ dy, const int32_t* __restrict__ offsets,
                                          int E, int rows, int f, int d,
                                          const float* __restrict__ Wd, const float* __restrict__ h,
                                          const float* __restrict__ u, float* __restrict__ dhu) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * f) return;
  const int r = (int)(i / f), n = (int)(i - (size_t)r * f);
  const int e = expert_of_row_b(offsets, E, r);
  const float* a = dy + (size_t)r * d;
  const float* w = Wd + ((size_t)e * f + n) * d;
  float acc = 0.f;
  for (int k = 0; k < d; ++k) acc = fmaf(a[k], w[k], acc);
  const float hv = h[i], uv = u[i];
  const float sg = 1.f / (1.f + __expf(-hv));
  dhu[(size_t)r * 2 * f + n] = acc * uv * sg * (1.f + hv * (1.f - sg));
  dhu[(size_t)r * 2 * f + f + n] = acc * hv * sg;
}

// dX[r, n] (+)= sum_{k < f} dhu[r, k] W_gate[e][n, k] + sum_{k < f} dhu[r, f + k] W_up[e][n, k]
__global__ void up_bwd_dgrad_f32_kernel(const float* __restrict__ dhu, const int32_t* __restrict__ offsets,
                                        int E, int rows, int d, int f,
                                        const float* __restrict__ Wg, const float* __restrict__ Wu,
                                        float* __restrict__ dx, int accumulate) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * d) return;
  const int r = (int)(i / d), n = (int)(i - (size_t)r * d);
  const int e = expert_of_row_b(offsets, E, r);
  const float* g = dhu + (size_t)r * 2 * f;
  const float* wg = Wg + ((size_t)e * d + n) * f;
  const float* wu = Wu + ((size_t)e * d + n) * f;
  float acc = 0.f;
  for (int k = 0; k < f; ++k) acc = fmaf(g[k], wg[k], acc);
  for (int k = 0; k < f; ++k) acc = fmaf(g[f + k], wu[k], acc);
  dx[i] = accumulate ? dx[i] + acc : acc;
}

// C_e[m, n] = sum_{r in e} A[src(r), m] B[r, n] (rows of e in order); columns
// n < n_split go to w0 [E, M, n_split], the rest to w1 [E, M, N - n_split]
__global__ void wgrad_f32_kernel(const float* __restrict__ A, int lda, const int32_t* __restrict__ gather,
                                 const float* __restrict__ B, int ldb,
                                 const int32_t* __restrict__ offsets, int E, int M, int N,
                                 int n_split, float* __restrict__ w0, float* __restrict__ w1) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)E * M * N) return;
  const int e = (int)(i / ((size_t)M * N));
  const size_t mn = i - (size_t)e * M * N;
  const int m = (int)(mn / N), n = (int)(mn - (size_t)m * N);
  float acc = 0.f;
  for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
    const int src = gather ? gather[r] : r;
    acc = fmaf(A[(size_t)src * lda + m], B[(size_t)r * ldb + n], acc);
  }
  if (n < n_split)
    w0[((size_t)e * M + m) * n_split + n] = acc;
  else
    w1[((size_t)e * M + m) * (N - n_split) + (n - n_split)] = acc;
}

unsigned blocks_of(size_t n) { return (unsigned)((n + 255) / 256); }

// dW_e = sum over the K chunks c (in order) of part[e][c] (M x N each), to
// w0 (columns < n_split) / w1; 4 columns per thread (N, n_split multiples of 8)
__global__ void wgrad_sum_kernel(const float* __restrict__ part, int E, int S, int M, int N,
                                 int n_split, float* __restrict__ w0, float* __restrict__ w1) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // 4-column group
  const size_t nv = (size_t)E * M * (N / 4);
  if (i >= nv) return;
  const int e = (int)(i / ((size_t)M * (N / 4)));
  const size_t rem = i - (size_t)e * M * (N / 4);
  const int m = (int)(rem / (N / 4)), n = (int)(rem - (size_t)m * (N / 4)) * 4;
  const size_t mn = (size_t)M * N;
  const float* src = part + (size_t)e * S * mn + (size_t)m * N + n;
  f32x4 acc = *reinterpret_cast<const f32x4*>(src);
  for (int c = 1; c < S; ++c) acc += *reinterpret_cast<const f32x4*>(src + (size_t)c * mn);
  float* dst = n < n_split ? w0 + ((size_t)e * M + m) * n_split + n
                           : w1 + ((size_t)e * M + m) * (N - n_split) + (n - n_split);
  __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(dst));
}

int pad8(long long g) { return (int)((g + 7) / 8 * 8); }

// DGRAD / WGRAD launches of the ping-pong kernel (tile 256 x 256)
// the ping-pong DGRAD keeps 32-bit element offsets of a tile's rows
bool dgrad256_ok(const BwdArgs& p) {
  return 256ll * (p.lda > p.K0 ? p.lda : p.K0) < (1ll << 31) &&
         (p.B1 == nullptr || p.K1 == p.K0);
}

// one launch for a layer's DGRAD and WGRAD only while the data gradient has
// at most this many rounds of tiles on the compute units (more measured slower)
constexpr int kPairMaxRounds = 12;

// grids of the 256 x 256 kernel (padded to a multiple of 8); they set the
// tile counts in the arguments
int dgrad256_grid(BwdArgs& p, int rows) {
  p.tiles_n = cdiv(p.N, 256);
  // sum_e ceil(c_e / 256) <= floor((rows + E (256 - 1)) / 256)
  const long long mt = ((long long)rows + (long long)p.E * 255) / 256;
  return pad8(mt * p.tiles_n);
}
int wgrad256_grid(BwdArgs& q) {
  q.tiles_m = cdiv(q.M, 256);
  q.tiles_n = cdiv(q.N, 256);
  return pad8((long long)q.E * q.ksplit * q.tiles_m * q.tiles_n);
}
bool dgrad_fast(const BwdArgs& p) { return p.K % 64 == 0 && p.K0 % 64 == 0; }
// the scalar-base form keeps 32-bit offsets within 32 rows of A and B
bool wgrad_fast(const BwdArgs& q) {
  return 32ll * (q.lda > q.ldb ? q.lda : q.ldb) * 2 < (1ll << 32);
}

// K chunks per expert for the weight gradients: when the launch has fewer
// than two tiles per compute unit (few experts: the shared experts run as one
// expert over every token), each expert's rows are cut into chunks of at least
// 512 rows so that about two tiles per compute unit run; the partials need
// E * S * M * N fp32 of workspace (with less, fewer chunks or none).
int wgrad_chunks(int E, int rows, int M, int N, size_t ws_bytes) {
  const long long tiles = (long long)E * cdiv(M, 256) * cdiv(N, 256);
  const long long want = 2ll * device_cu_count();
  if (tiles >= want || E <= 0) return 1;
  long long S = (want + tiles - 1) / tiles;
  S = std::min<long long>(S, std::max<long long>(1, (long long)rows / E / 512));
  S = std::min<long long>(S, 16);
  const long long per = (long long)E * M * N * 4;
  if (per > 0) S = std::min<long long>(S, (long long)(ws_bytes / per));
  return S >= 2 ? (int)S : 1;
}

void launch_wgrad_sum(const BwdArgs& q, hipStream_t s) {
  const size_t nv = (size_t)q.E * q.M * (q.N / 4);
  hipLaunchKernelGGL(wgrad_sum_kernel, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, s, q.part,
                     q.E, q.ksplit, q.M, q.N, q.n_split, q.w0, q.w1);
}

template <int EPI>
void launch_dgrad256(BwdArgs p, int rows, hipStream_t s) {
  const int grid = dgrad256_grid(p, rows);
  if (grid <= 0) return;
  if (dgrad_fast(p))
    hipLaunchKernelGGL((grouped_gemm_bwd256_kernel<DGRAD, EPI, true>), dim3(grid), dim3(512), 0, s,
                       p);
  else
    hipLaunchKernelGGL((grouped_gemm_bwd256_kernel<DGRAD, EPI>), dim3(grid), dim3(512), 0, s, p);
}
// the kernel's view of a WGRAD launch: with a K split, the partials go to
// slabs of the workspace (one M x N slab per expert and chunk)
BwdArgs wgrad_kernel_args(const BwdArgs& q) {
  BwdArgs g = q;
  if (q.ksplit > 1) {
    g.w0 = q.part;
    g.w1 = nullptr;
    g.n_split = q.N;
  }
  return g;
}
void launch_wgrad256(BwdArgs q, hipStream_t s) {
  const int grid = wgrad256_grid(q);
  const BwdArgs g = wgrad_kernel_args(q);
  if (wgrad_fast(q))
    hipLaunchKernelGGL((grouped_gemm_bwd256_kernel<WGRAD, EPI_WGRAD, true>), dim3(grid), dim3(512), 0,
                       s, g);
  else
    hipLaunchKernelGGL((grouped_gemm_bwd256_kernel<WGRAD, EPI_WGRAD>), dim3(grid), dim3(512), 0, s,
                       g);
  if (q.ksplit > 1) launch_wgrad_sum(q, s);
}

// DGRAD and WGRAD of one layer in one launch when both take the scalar-base
// 256 x 256 kernel; returns false (nothing launched) otherwise
template <int EPI>
bool launch_pair256(BwdArgs p, BwdArgs q, int rows, hipStream_t s) {
  if (rows <= 0 || !dgrad256_ok(p) || !dgrad_fast(p) || q.a_gather != nullptr || !wgrad_fast(q))
    return false;
  const int gd = dgrad256_grid(p, rows);
  // only where the data gradient has few rounds of tiles, so that its last,
  // partial round matters (typical tiles: rows / 256 + E / 2 per N panel).
  // Measured: a 2.4-round layer gains 8%, 8.3 rounds 1.4%; at 16 and 25
  // rounds the pair was 1-4% slower than two launches.
  const long long typ = ((long long)rows / 256 + p.E / 2) * p.tiles_n;
  if (typ > (long long)kPairMaxRounds * device_cu_count()) return false;
  const int gw = wgrad256_grid(q);
  hipLaunchKernelGGL((grouped_gemm_bwd256_pair_kernel<EPI>), dim3(gd + gw), dim3(512), 0, s, p,
                     wgrad_kernel_args(q), gd);
  if (q.ksplit > 1) launch_wgrad_sum(q, s);
  return true;
}

int dgrad_grid(int rows, int E, int tiles_n) {
  // sum_e ceil(c_e / BM) <= floor((rows + E (BM - 1)) / BM)
  const long long mt = ((long long)rows + (long long)E * (BM - 1)) / BM;
  return (int)(mt * tiles_n);
}

}  // namespace

size_t ffn_backward_workspace_bytes(int E, int rows, int d, int f) {
  const size_t huge = (size_t)1 << 62;
  const int s1 = wgrad_chunks(E, rows, f, d, huge);      // dW_down: M = f, N = d
  const int s0 = wgrad_chunks(E, rows, d, 2 * f, huge);  // dW_gate | dW_up: M = d, N = 2f
  const size_t b1 = s1 > 1 ? (size_t)E * s1 * f * d * 4 : 0;
  const size_t b0 = s0 > 1 ? (size_t)E * s0 * d * 2 * f * 4 : 0;
  return align_up(b1 > b0 ? b1 : b0, 256);
}

hipError_t launch_expert_down_backward(const void* dy_perm, const int32_t* offsets, int E,
                                       int rows, int f, int d, bool bf16, const void* W_down,
                                       const void* h, const void* u, const void* act,
                                       void* dhu, float* dW_down, void* ws, size_t ws_bytes,
                                       hipStream_t s) {
  if (!bf16) {
    if (rows > 0)
      hipLaunchKernelGGL(down_bwd_dgrad_f32_kernel, dim3(blocks_of((size_t)rows * f)), dim3(256),
                         0, s, static_cast<const float*>(dy_perm), offsets, E, rows, f, d,
                         static_cast<const float*>(W_down), static_cast<const float*>(h),
                         static_cast<const float*>(u), static_cast<float*>(dhu));
    hipLaunchKernelGGL(wgrad_f32_kernel, dim3(blocks_of((size_t)E * f * d)), dim3(256), 0, s,
                       static_cast<const float*>(act), f, nullptr,
                       static_cast<const float*>(dy_perm), d, offsets, E, f, d, d, dW_down,
                       nullptr);
    return hipGetLastError();
  }
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
  q.ksplit = wgrad_chunks(E, rows, f, d, ws_bytes);
  q.part = static_cast<float*>(ws);
  if (launch_pair256<EPI_SWIGLU_BWD>(p, q, rows, s)) return hipGetLastError();
  if (rows > 0) {
    if (dgrad256_ok(p)) {
      launch_dgrad256<EPI_SWIGLU_BWD>(p, rows, s);
    } else {
      const int grid = dgrad_grid(rows, E, p.tiles_n);
      if (grid > 0)
        hipLaunchKernelGGL((grouped_gemm_bwd_kernel<DGRAD, EPI_SWIGLU_BWD>), dim3(grid), dim3(NT),
                           0, s, p);
    }
  }
  launch_wgrad256(q, s);
  return hipGetLastError();
}

hipError_t launch_expert_up_backward(const void* x, const int32_t* gather_idx,
                                     const int32_t* offsets, int E, int rows, int d, int f,
                                     bool bf16, const void* W_gate, const void* W_up,
                                     const void* dhu, float* dx_perm, int accumulate,
                                     float* dW_gate, float* dW_up, void* ws, size_t ws_bytes,
                                     hipStream_t s) {
  if (!bf16) {
    if (rows > 0)
      hipLaunchKernelGGL(up_bwd_dgrad_f32_kernel, dim3(blocks_of((size_t)rows * d)), dim3(256), 0,
                         s, static_cast<const float*>(dhu), offsets, E, rows, d, f,
                         static_cast<const float*>(W_gate), static_cast<const float*>(W_up),
                         dx_perm, accumulate);
    hipLaunchKernelGGL(wgrad_f32_kernel, dim3(blocks_of((size_t)E * d * 2 * f)), dim3(256), 0, s,
                       static_cast<const float*>(x), d, gather_idx,
                       static_cast<const float*>(dhu), 2 * f, offsets, E, d, 2 * f, f, dW_gate,
                       dW_up);
    return hipGetLastError();
  }
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
  // the K split needs the 256 x 256 kernel (rows in order, no gather)
  q.ksplit = gather_idx == nullptr ? wgrad_chunks(E, rows, d, 2 * f, ws_bytes) : 1;
  q.part = static_cast<float*>(ws);
  const bool add = accumulate != 0;
  if (add ? launch_pair256<EPI_F32_ADD>(p, q, rows, s) : launch_pair256<EPI_F32>(p, q, rows, s))
    return hipGetLastError();
  if (rows > 0) {
    if (dgrad256_ok(p)) {
      if (add)
        launch_dgrad256<EPI_F32_ADD>(p, rows, s);
      else
        launch_dgrad256<EPI_F32>(p, rows, s);
    } else {
      const int grid = dgrad_grid(rows, E, p.tiles_n);
      if (grid > 0)
        hipLaunchKernelGGL((grouped_gemm_bwd_kernel<DGRAD, EPI_F32>), dim3(grid), dim3(NT), 0, s,
                           p);
    }
  }
  if (gather_idx == nullptr)  // the ping-pong WGRAD reads A rows in order
    launch_wgrad256(q, s);
  else
    hipLaunchKernelGGL((grouped_gemm_bwd_kernel<WGRAD, EPI_WGRAD>),
                       dim3((unsigned)(E * q.tiles_m * q.tiles_n)), dim3(NT), 0, s, q);
  return hipGetLastError();
}

}  // namespace moe
