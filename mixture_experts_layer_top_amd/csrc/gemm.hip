// Grouped expert GEMMs: "layer 0" (gate/up projections with fused SwiGLU)
// and "layer 1" (down projection with optional fused weighted combine).
//
// The two GEMMs of an expert and their decomposition: COMET page, "COMET's
// Technical Principles" -- layer 0 split along the token dimension M,
// layer 1 along the hidden dimension N, chosen there so that communication
// and computation units line up across GPUs.  On one GPU there is nothing
// to line up, and the tile walk is chosen for the caches instead: both
// layers walk M fastest inside an (expert, weight panel), so the tiles that
// run together share the panel.
//
// bf16 kernels (gfx950), both with 256-row x 256-accumulator-column tiles,
// K stages of 64, v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
//   * grouped_gemm_bf16_pp_kernel (K a multiple of 64, the token operand
//     below 4 GiB): 8 waves in two groups of 4, X (rows 0-127) and Y (rows
//     128-255), taking turns on the matrix cores ("ping-pong"): while one
//     group runs its MFMAs at raised priority, the other reads its fragments
//     of the next stage from LDS and issues its share of the operand loads
//     (X all A loads, Y all B loads), with a workgroup barrier between
//     phases.  LDS holds an A ring of 2 stages and a B ring of 3 (5 x 32 KiB);
//   * grouped_gemm_bf16_kernel (any K a multiple of 8, any operand size):
//     8 waves that all load and all compute, the K tail zero-filled on load;
//   * layer 0: the 256 columns are 128 columns of W_gate and the same 128 of
//     W_up, so SiLU(h) * u is formed in registers; its rows are gathered on
//     load through the permutation, so no permuted copy of x exists;
//   * layer 1 writes fp32 rows, or compact rows (fp16 with a power-of-two
//     factor per 32-column segment, store_seg_f16), or adds w * out into y
//     with atomics (the fused combine);
//   * operands move HBM -> LDS with global_load_lds_dwordx4 (no register
//     staging); one load fills 1 KiB of consecutive LDS, so each layout's
//     swizzle is applied to the global addresses; A (K contiguous) is read
//     with ds_read_b128, B (the caller's [K, N] weights, N contiguous) with
//     ds_read_b64_tr_b16, the gfx950 LDS transpose read: no repacked copy;
//   * tiles never straddle experts; each workgroup derives its tile from the
//     device offsets (a wave prefix sum by DPP), so the host never reads the
//     routing; tiles go M fastest inside an (expert, weight panel), large
//     experts in groups of M tiles whose rows stay in the last-level cache,
//     and consecutive tiles land on one XCD (its L2); an expert's rows are
//     dealt to its M tiles in balanced 16-row blocks; the last round's tiles
//     are split along K when it is mostly idle, and a second launch adds the
//     parts in order (deterministic);
//   * wide items (K of 2048 and more): an expert whose last rows fill at most
//     half a tile takes whole 256-row tiles for the rest, and those last rows
//     as one item per pair of N panels, both groups on the same rows, X on
//     one panel and Y on the next (rings of 2, 16 + 64 KiB a stage): a
//     nearly empty tile per panel becomes half an item.  Every output
//     element sees the same K order either way (same bits).
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 256;        // rows per tile
constexpr int BK = 64;         // K per pipeline stage
constexpr int A_CPR = BK / 8;    // 16-byte chunks per A row in a stage
constexpr int A_RPL = 1024 / (BK * 2);  // A rows per 1 KiB load
constexpr int A_LOADS = BM * BK * 2 / 1024;
// LDS stage buffers: two for the token operand (A), three for the weight
// operand (B), 2 x 32 + 3 x 32 = 160 KiB: weight loads are issued two
// stages ahead, token rows one stage ahead
constexpr int A_SLOTS = 2, B_SLOTS = 3;
constexpr int A_BYTES = BM * BK * 2;  // 32 KiB per stage

// Per tile-width constants.  BNA = accumulator columns per tile.
template <int BNA>
struct TileCfg {
  static constexpr int B_BYTES = BK * BNA * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int CPR = BNA / 8;                     // 16-byte chunks per B row
  static constexpr int ROWS_PER_LOAD = 1024 / (BNA * 2);  // B rows per 1 KiB load
  static constexpr int B_LOADS = B_BYTES / 1024;
};

struct GemmArgs {
  const bf16_t* A;          // [n_a, K] rows (x for layer 0, activations for layer 1)
  const int32_t* gather;    // row r reads A[gather[r]] (layer 0) or NULL
  const int32_t* offsets;   // [E+1]
  int E, rows, K, N;
  const bf16_t* B0;         // [E, K, N]: W_gate (layer 0) or W_down (layer 1)
  const bf16_t* B1;         // [E, K, N]: W_up (layer 0) or NULL
  bf16_t* a_out;            // layer 0 output [rows, N]
  bf16_t* h_out;            // layer 0: x W_gate [rows, N] saved for the backward, or NULL
  bf16_t* u_out;            // layer 0: x W_up [rows, N] (given with h_out)
  float* y_perm;            // layer 1 output [rows, N] or NULL
  uint16_t* y_h;            // layer 1 compact output [rows, N] fp16, or NULL (see store_seg_f16)
  float* y_s;               // its restoring factors [rows, N / 32] (with y_h)
  const int32_t* scatter;   // layer 1 fused combine target row, or NULL (identity)
  const float* row_w;       // layer 1 fused combine weight, or NULL (1)
  float* y;                 // layer 1 fused combine target, or NULL
  int tiles_n;              // column tiles per expert
  int grid_per_xcd;         // padded grid / 8
  int m_group;              // ping-pong kernel: most M tiles walked per pass over the N panels
  int m_group_min;          // experts with at most this many M tiles are walked in one pass
  // ping-pong kernel only: tail split (see assign_work)
  float* part;              // partial accumulators of split tiles, or NULL (no split)
  int n_cu;                 // compute units the tiles are spread over
  int fixup;                // 0: main pass; 1: sum the split tiles' partials
  int nt_y;                 // layer-1 output stores non-temporal (larger than the last-level cache)
  int wide_rem;             // 1: an expert's last rows, when at most BM / 2, form wide items
};

// Compact layer-1 output: IEEE fp16 with one power-of-two factor per
// 32-column row segment.  The segment's largest finite magnitude m is scaled
// into [2^14, 2^15), well inside the fp16 range, so nothing overflows and
// every value keeps fp16's 11 significant bits at the segment's scale
// (round to nearest even; relative error at most 2^-11 of the segment's
// largest value); y_s holds the factor that restores it, 1 / scale, exact
// since both are powers of two.  Inf and NaN do not set the scale and stay
// inf and NaN.  Four consecutive lanes hold one segment, 8 columns each:
// src (LDS, 8 floats), dst (8 columns of y_h), fdst (the segment's factor,
// written by the first lane of the four); valid: the lane's row and columns
// exist.  Every lane of the wave must take part (quad reduction by DPP).
template <bool NT>
__device__ __forceinline__ void store_seg_f16v(const f32x4 a, const f32x4 b, uint16_t* dst,
                                               float* fdst, bool valid, bool leader) {
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t m = 0;  // largest finite magnitude, as bits (ordered like the values)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t u = __float_as_uint(v[i]) & 0x7fffffffu;
    m = max(m, u < 0x7f800000u ? u : 0u);
  }
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));  // lane ^ 1
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));  // lane ^ 2
  // m lies in [2^(eb - 127), 2^(eb - 126)); the scale 2^(141 - eb) takes it
  // into [2^14, 2^15).  eb is raised to at least 15 so that scale and factor
  // are normal floats (segments below 2^-112 are stored as they are scaled).
  const int eb = max((int)(m >> 23), 15);
  const float scale = __uint_as_float((uint32_t)(268 - eb) << 23);
  const float back = __uint_as_float((uint32_t)(eb - 14) << 23);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 lo = static_cast<_Float16>(v[2 * i] * scale);
    const _Float16 hi = static_cast<_Float16>(v[2 * i + 1] * scale);
    o[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
  }
  if (valid) {
    if (NT) {
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst));
      if (leader) __builtin_nontemporal_store(back, fdst);
    } else {
      *reinterpret_cast<u32x4*>(dst) = o;
      if (leader) *fdst = back;
    }
  }
}
template <bool NT>
__device__ __forceinline__ void store_seg_f16(const float* src, uint16_t* dst, float* fdst,
                                              bool valid, bool leader) {
  store_seg_f16v<NT>(*reinterpret_cast<const f32x4*>(src), *reinterpret_cast<const f32x4*>(src + 4),
                     dst, fdst, valid, leader);
}

struct TileInfo {
  int e, row0, row_end, n_t, m_t;
  int nb;     // ping-pong kernel: 16-row blocks in the tile (<= BM / 16)
  bool wide;  // ping-pong kernel: at most BM / 2 rows over N panels n_t and n_t + 1
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
  const int incl = wave_incl_sum(lane_sum);
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
  const int src = __ffsll((unsigned long long)hit) - 1;  // uniform: read from that lane
  ti.e = __builtin_amdgcn_readlane(hit_e, src);
  const int tstart = __builtin_amdgcn_readlane(hit_start, src);
  const int tmt = __builtin_amdgcn_readlane(hit_mt, src);
  const int toff = __builtin_amdgcn_readlane(hit_off, src);
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

// Byte offsets inside one stage.
// A: [BM rows][BK] bf16, 2 BK bytes per row.  A fragment read touches 16
// consecutive rows at one 16-byte chunk.  The chunk index is XOR-ed with
// (row >> 1) & 7, measured free of bank conflicts on gfx950.
// B: [BK rows][BNA] bf16.  One transpose read touches 4 rows x 32 bytes per
// 16 lanes (rows 8 apart for the next 16 lanes).  The chunk index is XOR-ed
// with 2 * (row % 8) + (row & 8): even values keep the 32-byte pairs whole,
// the low part spreads 4 rows over a 128-byte window and bit 3 moves rows
// 8..15 to the other half of a 256-byte window.
__device__ __forceinline__ int a_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int a_off(int row, int chunk) {
  return row * (BK * 2) + ((chunk ^ a_swz(row)) << 4);
}
template <int BNA>
__device__ __forceinline__ int b_swz(int krow) {
  constexpr int CPR = BNA / 8;  // 16 or 32 chunks per row
  return (((krow & 7) << 1) + (krow & 8)) & (CPR - 1);
}
template <int BNA>
__device__ __forceinline__ int b_off(int krow, int col) {
  return krow * (BNA * 2) + (((col >> 3) ^ b_swz<BNA>(krow)) << 4) + ((col & 7) << 1);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// 16 zero bytes in device memory: A chunks past K load from here, so the
// K tail of the last stage arrives as zeros (no clearing pass needed).
__device__ __attribute__((aligned(16))) const bf16_t kZeroChunk[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// One direct-to-LDS load: 64 lanes x 16 bytes from their global addresses to
// the 1 KiB of LDS starting at lds_addr (wave-uniform).  Written as inline
// assembly so that the compiler's wait-count pass does not model it: these
// loads are waited for explicitly with wait_vmcnt (the main loop issues no
// other vector-memory operation, and its last stage waits for zero).
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_addr) {
  // no "memory" clobber: the compiler would then wait for all vector-memory
  // operations before every later LDS read.  Ordering against the LDS reads
  // of the same buffer comes from s_barrier, which the compiler does not
  // move volatile statements across.
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "s"(lds_addr)
      : "m0");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// WM x WN waves; each owns (BM / WM) x (BNA / WN) accumulators.
template <bool UP, int WM, int WN, int BNA>
__global__ __launch_bounds__(64 * WM * WN, 1) void grouped_gemm_bf16_kernel(GemmArgs p) {
  using C = TileCfg<BNA>;
  constexpr int NW = WM * WN;
  constexpr int MI = BM / WM / 16;     // 16-row blocks per wave
  constexpr int NJ = BNA / WN / 16;    // 16-column blocks per wave
  constexpr int A_LD = A_LOADS / NW;   // A loads per wave per stage
  constexpr int B_LD = C::B_LOADS / NW;
  static_assert(A_LD >= 1 && B_LD >= 1 && A_LOADS % NW == 0 && C::B_LOADS % NW == 0,
                "loader split");
  static_assert(!UP || NJ % 2 == 0, "gate/up pairs");
  constexpr int LDS_OPS = A_SLOTS * A_BYTES + B_SLOTS * C::B_BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_OPS];
  // operand buffers: A slots first, then B slots
  auto a_base = [&](int kt) { return (kt % A_SLOTS) * A_BYTES; };
  auto b_base = [&](int kt) { return A_SLOTS * A_BYTES + (kt % B_SLOTS) * C::B_BYTES; };

  const int b = blockIdx.x;
  const int tile = (b & 7) * p.grid_per_xcd + (b >> 3);
  // both layers walk M fastest inside an (expert, N panel): the tiles that
  // run together on an XCD then share their weight panel (read once from
  // HBM) and a handful of token-row blocks (measured: higher L2 hit rate and
  // faster than walking N fastest for layer 1 too)
  const TileInfo ti = locate_tile<true>(p, tile);
  if (!ti.ok) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int K = p.K, N = p.N;
  const int n0 = ti.n_t * (UP ? BNA / 2 : BNA);
  const uint32_t lds0 = lds_addr_of(lds);
  const int nk = cdiv(K, BK);  // K stages (the last one zero-filled past K)

  // ---- direct-to-LDS loader.  One load moves 64 lanes x 16 B = 1 KiB into
  // consecutive LDS bytes, so each layout's swizzle is applied on the global
  // side: lane i fills slot i.  A load j: rows A_RPL j .. A_RPL (j + 1) - 1.
  const bf16_t* a_src[A_LD];
  int a_k[A_LD];  // this lane's K offset inside a stage
#pragma unroll
  for (int q = 0; q < A_LD; ++q) {
    const int row = (wave * A_LD + q) * A_RPL + lane / A_CPR;
    a_k[q] = ((lane % A_CPR) ^ a_swz(row)) * 8;
    int r = ti.row0 + row;
    if (r >= ti.row_end) r = ti.row0;  // padding rows read a valid row; results are discarded
    const int src_row = p.gather ? p.gather[r] : r;
    a_src[q] = p.A + (size_t)src_row * K;
  }
  // B load j: K rows j * ROWS_PER_LOAD ..
  const bf16_t* b_src[B_LD];
  int b_krow[B_LD];
#pragma unroll
  for (int q = 0; q < B_LD; ++q) {
    const int krow = (wave * B_LD + q) * C::ROWS_PER_LOAD + lane / C::CPR;
    const int chunk = (lane % C::CPR) ^ b_swz<BNA>(krow);
    const bf16_t* mat;
    int col;
    if (UP) {
      mat = (chunk < C::CPR / 2) ? p.B0 : p.B1;
      col = n0 + (chunk % (C::CPR / 2)) * 8;
    } else {
      mat = p.B0;
      col = n0 + chunk * 8;
    }
    if (col >= N) col = N - 8;  // padding columns read valid data; results are discarded
    b_krow[q] = krow;
    b_src[q] = mat + (size_t)ti.e * K * N + col;
  }
  // load i (0 <= i < A_LD + B_LD) of this wave's share of a stage: the A
  // loads (i < A_LD) of stage kt_a, the B loads of stage kt_b; stages past
  // the last are skipped
  auto issue_load2 = [&](int kt_a, int kt_b, int i) {
    if (i < A_LD) {
      if (kt_a >= nk) return;
      const int kk = kt_a * BK + a_k[i];
      const bf16_t* src = kk < K ? a_src[i] + kk : kZeroChunk;  // K tail -> zeros
      lds_dma16(src, lds0 + (uint32_t)(a_base(kt_a) + (wave * A_LD + i) * 1024));
    } else {
      if (kt_b >= nk) return;
      const int q = i - A_LD;
      const int kr = min(kt_b * BK + b_krow[q], K - 1);
      lds_dma16(b_src[q] + (size_t)kr * N,
                lds0 + (uint32_t)(b_base(kt_b) + (wave * B_LD + q) * 1024));
    }
  };

  // ---- per-lane LDS read offsets (within a stage)
  const int wrow0 = wm * (BM / WM);
  constexpr int KS = BK / 32;  // MFMA K steps per stage
  int a_rd[KS][MI];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      a_rd[ks][mi] = a_off(wrow0 + mi * 16 + (lane & 15), ks * 4 + (lane >> 4));
  auto col_block = [&](int nj) {
    if (UP)
      return (nj < NJ / 2) ? (wn * (NJ / 2) * 16 + nj * 16)
                           : (BNA / 2 + wn * (NJ / 2) * 16 + (nj - NJ / 2) * 16);
    return wn * NJ * 16 + nj * 16;
  };
  int b_rd[KS][NJ], b_rd4[KS][NJ];
  const int b_kr = (lane >> 4) * 8 + ((lane & 15) >> 2);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
      // rows b_kr and b_kr + 4 differ in their swizzle: separate offsets
      b_rd[ks][nj] = b_off<BNA>(ks * 32 + b_kr, col_block(nj) + (lane & 3) * 4);
      b_rd4[ks][nj] = b_off<BNA>(ks * 32 + b_kr + 4, col_block(nj) + (lane & 3) * 4);
    }

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto read_frags = [&](int kt, int ks, bf16x8 (&af)[MI], bf16x8 (&bfr)[NJ]) {
    const char* As = lds + a_base(kt);
    const char* Bs = lds + b_base(kt);
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Bs + b_rd[ks][nj]));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Bs + b_rd4[ks][nj]));
      bfr[nj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) af[mi] = *reinterpret_cast<const bf16x8*>(As + a_rd[ks][mi]);
  };
  auto mfmas = [&](const bf16x8 (&af)[MI], const bf16x8 (&bfr)[NJ]) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj)
        acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[nj], acc[mi][nj], 0, 0, 0);
  };
  // the same MFMAs with the loads of A(ld_a) and B(ld_b) spread between
  // their rows, so that no wave stalls on a burst of load issues while its
  // matrix core idles
  auto mfmas_with_loads = [&](const bf16x8 (&af)[MI], const bf16x8 (&bfr)[NJ], int ld_a,
                              int ld_b) {
    constexpr int NL = A_LD + B_LD;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj)
        acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[nj], acc[mi][nj], 0, 0, 0);
      // loads i with i * MI / NL == mi go after row mi (A loads first)
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if ((i * MI) / NL == mi) issue_load2(ld_a, ld_b, i);
    }
  };

  // prologue: B(0), then the steady-state group [A(0), B(1)]
#pragma unroll
  for (int i = A_LD; i < A_LD + B_LD; ++i) issue_load2(0, 0, i);
#pragma unroll
  for (int i = 0; i < A_LD + B_LD; ++i) issue_load2(0, 1, i);
  for (int kt = 0; kt < nk; ++kt) {
    // A(kt) and B(kt) have landed once at most B(kt + 1) is outstanding;
    // then every wave's share is visible after the barrier, and every wave
    // is done with the buffers of stage kt - 1
    if (kt + 1 < nk) wait_vmcnt<B_LD>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    bf16x8 af[MI], bfr[NJ];
    read_frags(kt, 0, af, bfr);
    // A(kt + 1) into the A slot of stage kt - 1, B(kt + 2) into the B slot
    // of stage kt - 1: both were last read before this stage's barrier
    mfmas_with_loads(af, bfr, kt + 1, kt + 2);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) {
      read_frags(kt, ks, af, bfr);
      mfmas(af, bfr);
    }
  }
  wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup ends

  // ---- epilogue.  Accumulator layout of a 16 x 16 block: column lane % 16,
  // rows 4 * (lane / 16) + i.  Outputs go through a per-wave LDS staging
  // area (16 rows at a time) so that global stores are 16-byte vectors
  // covering whole row segments.
  __syncthreads();  // every wave is done reading the operand stages
  const int col_l = lane & 15;
  const int row_l = (lane >> 4) * 4;
  // per-wave staging area: 16 rows of the wave's output columns, padded
  constexpr int STG = UP ? 16 * (NJ / 2 * 16 + 8) * 2 : 16 * (NJ * 16 + 4) * 4;
  static_assert(STG % 16 == 0 && NW * STG <= LDS_OPS, "staging fits the operand LDS");
  char* stg = lds + wave * STG;
  if (UP) {
    // 16 rows x (NJ / 2 * 16) bf16 outputs per block row; the wave's output
    // columns are contiguous: n0 + wn * (NJ / 2) * 16 + [0, NJ / 2 * 16)
    constexpr int OC = NJ / 2 * 16;          // output columns per wave
    constexpr int SS = OC + 8;               // staging stride in bf16 (16-byte aligned)
    bf16_t* sb = reinterpret_cast<bf16_t*>(stg);
    const int ocol0 = n0 + wn * OC;
    const int nout = p.h_out ? 3 : 1;  // SiLU(h) u, then (training) h and u
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      for (int o = 0; o < nout; ++o) {
        bf16_t* dst = o == 0 ? p.a_out : (o == 1 ? p.h_out : p.u_out);
#pragma unroll
        for (int nj = 0; nj < NJ / 2; ++nj)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float h = acc[mi][nj][i], u = acc[mi][nj + NJ / 2][i];
            sb[(row_l + i) * SS + nj * 16 + col_l] = f32_to_bf16(o == 0 ? silu(h) * u : (o == 1 ? h : u));
          }
        // each lane stores 16 bytes (8 columns) of one row
        constexpr int CH = OC / 8;              // 16-byte chunks per row
#pragma unroll
        for (int q = 0; q < (16 * CH + 63) / 64; ++q) {
          const int idx = q * 64 + lane;
          if (idx < 16 * CH) {
            const int r = idx / CH, c = idx % CH;
            const int row = ti.row0 + wrow0 + mi * 16 + r;
            const int col = ocol0 + c * 8;
            const u32x4 v = *reinterpret_cast<const u32x4*>(sb + r * SS + c * 8);
            if (row < ti.row_end && col < N)
              *reinterpret_cast<u32x4*>(dst + (size_t)row * N + col) = v;
          }
        }
      }
    }
  } else {
    if (p.y_perm || p.y_h) {
      constexpr int OC = NJ * 16;   // output columns per wave, contiguous
      constexpr int SS = OC + 4;    // staging stride in floats (16-byte aligned, padded)
      float* sf = reinterpret_cast<float*>(stg);
      const int ocol0 = n0 + wn * OC;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
          for (int i = 0; i < 4; ++i) sf[(row_l + i) * SS + nj * 16 + col_l] = acc[mi][nj][i];
        if (p.y_h) {
          // 16 rows x OC / 8 chunks of 8 columns; OC is a multiple of 32 and
          // the wave's columns start at a multiple of 32 (N too): whole segments
          static_assert(OC % 32 == 0 && (16 * OC / 8) % 64 == 0, "compact output segments");
          constexpr int CH = OC / 8;
          const int segs = N >> 5;
#pragma unroll
          for (int q = 0; q < 16 * CH / 64; ++q) {
            const int idx = q * 64 + lane;
            const int r = idx / CH, c = idx % CH;
            const int row = ti.row0 + wrow0 + mi * 16 + r;
            const int col = ocol0 + c * 8;
            store_seg_f16<false>(sf + r * SS + c * 8, p.y_h + (size_t)row * N + col,
                                 p.y_s + (size_t)row * segs + (col >> 5),
                                 row < ti.row_end && col < N, (c & 3) == 0);
          }
          continue;
        }
        constexpr int CH = OC / 4;  // 16-byte chunks per row
#pragma unroll
        for (int q = 0; q < (16 * CH + 63) / 64; ++q) {
          const int idx = q * 64 + lane;
          if (idx < 16 * CH) {
            const int r = idx / CH, c = idx % CH;
            const int row = ti.row0 + wrow0 + mi * 16 + r;
            const int col = ocol0 + c * 4;
            const f32x4 v = *reinterpret_cast<const f32x4*>(sf + r * SS + c * 4);
            if (row < ti.row_end && col < N)
              *reinterpret_cast<f32x4*>(p.y_perm + (size_t)row * N + col) = v;
          }
        }
      }
    }
    if (p.y) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = ti.row0 + wrow0 + mi * 16 + row_l + i;
          if (row >= ti.row_end) continue;
          const int tgt = p.scatter ? p.scatter[row] : row;
          float* yrow = p.y + (size_t)tgt * N;
          const float wgt = p.row_w ? p.row_w[row] : 1.f;
#pragma unroll
          for (int nj = 0; nj < NJ; ++nj) {
            const int col = n0 + col_block(nj) + col_l;
            if (col < N) unsafeAtomicAdd(yrow + col, wgt * acc[mi][nj][i]);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// Ping-pong kernel: 8 wave64s, two per SIMD, in two groups that take turns
// on the SIMD's matrix core.  Group X (waves 0-3) owns rows 0-127 of the
// 256 x 256 macro tile, group Y (waves 4-7) rows 128-255; wave w of a group
// owns columns w * 32 + [0, 32) of both 128-column B halves (128 x 64 =
// 8 x 4 accumulator blocks).  Phases, separated by workgroup barriers:
//
//   phase 2s    : X memory(s)  | Y compute(s - 1)
//   phase 2s + 1: X compute(s) | Y memory(s)
//
// memory(s) = read the wave's fragments of stage s from LDS and issue the
// wave's loads of a later stage; compute(s) = its MFMAs on stage s.  So on
// every SIMD one wave keeps the matrix core busy while the other waits on
// LDS reads and load issue.  X issues all A loads, Y all B loads.  With
// rings of RA (A) and RB (B) stages, memory(s) loads stage s + RA - 1 (X)
// or s + RB - 1 (Y) into the slot of stage s - 1, whose readers finished
// before phase 2s (each memory phase ends with its reads waited for); a
// wave waits for its part of stage s + 1 at the end of phase 2s + 1, and
// the barrier after it makes the stage visible to all.
//
// Stage depth PBK = 64: two MFMA K steps per stage; rings of 2 (A) and 3
// (B) stages fill the 160 KiB of LDS (32-deep stages with rings of 5 + 5,
// which issue every load 3 stages ahead, measured slower: twice the
// barriers per K).
//
// B stage layout: two halves of PBK K rows x 128 columns (256 B per row),
// each 1 KiB load filling 4 rows of one half.  Layer 0: half 0 = W_gate,
// half 1 = W_up (the same 128 columns); layer 1: the two 128-column halves
// of a 256-column panel.
//
// Loads use the scalar-base form of global_load_lds_dwordx4 (uniform 64-bit
// base + per-lane 32-bit byte offset): one register per load slot; stages
// advance the scalar base.  K must be a multiple of PBK and the A operand
// smaller than 4 GiB; other shapes take the kernel above.
// ------------------------------------------------------------------------
namespace pp {
constexpr int NW = 8, MI = 8, NJ = 4;

template <int PBK>
struct Cfg {
  static constexpr int SLOT = BM * PBK * 2;            // one operand stage (A or B)
  static constexpr int HALF = PBK * 128 * 2;           // one B half
  static_assert(PBK == 64, "stage depth");
  static constexpr int RA = 2;                         // A ring
  static constexpr int RB = 3;                         // B ring
  static constexpr int LDS_BYTES = (RA + RB) * SLOT;
  static constexpr int KS = PBK / 32;                  // MFMA K steps per stage
  static constexpr int LD = SLOT / 1024 / 4;           // 1 KiB loads per wave per stage
  static constexpr int CPR = PBK / 8;                  // 16-byte chunks per A row
  static constexpr int RPL = 1024 / (PBK * 2);         // A rows per load
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// A swizzle: the 16-byte chunk index XOR-ed with row / 2 (mod chunks per
// row).  It depends on the row's position inside its 16-row block only,
// so every fragment block of a wave has the same lane offsets (one
// register plus immediates), and it makes the fragment read (16 rows at
// one chunk per 16 lanes) free of LDS bank conflicts on gfx950: measured
// with SQ_LDS_BANK_CONFLICT, 0 for 128-byte and 64-byte rows, against ~1
// conflict cycle per busy cycle for XOR with row % 8, row % 8 ^ row / 8,
// 2 (row / 4 % 4) (128-byte rows) or row / 4 % 4 (64-byte rows).
template <int PBK>
__device__ __forceinline__ int a_swz16(int row) { return (row >> 1) & (PBK / 8 - 1); }

// One direct-to-LDS load with a scalar base: lane i reads 16 bytes at
// base + voff_i and writes LDS bytes lds_addr + 16 i.
__device__ __forceinline__ void lds_dma16_s(uint32_t voff, const void* base, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "m0");
}

__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(n * LD) for a run-time n in 0..3
template <int LD>
__device__ __forceinline__ void wait_groups(int n) {
  if (n >= 3) wait_vmcnt<3 * LD>();
  else if (n == 2) wait_vmcnt<2 * LD>();
  else if (n == 1) wait_vmcnt<LD>();
  else wait_vmcnt<0>();
}
}  // namespace pp

// Tail split.  With N_t output tiles on C compute units the last round
// holds N_t mod C tiles; when that is at most C / 2 (and N_t <= 64 C), each
// of those tail tiles is split along K into S = min(C / tail, stages) parts
// that run side by side, their fp32 partial accumulators go to p.part, and a second
// launch (fixup) adds the parts in part order and runs the tile's normal
// epilogue.  Every workgroup derives N_t, the split and its own work item
// from the device offsets, so the host never reads the routing.
//   main pass, block b: b < G (the first F = N_t - tail tiles, padded to a
//     multiple of 8 and walked XCD-aware as usual) -> full tile; b >= G ->
//     split item j = b - G: tail tile F + j / S, part j % S;
//   fixup pass, block b < tail * FIXQ: tail tile F + b / FIXQ, 16-row
//     block b % FIXQ of each wave (the partials are read by FIXQ times more
//     workgroups than there are tail tiles).
constexpr int kSplitMaxRounds = 64;  // no tail split for launches of more rounds
constexpr int FIXQ = 8;  // fixup workgroups per tail tile (one 16-row block of each wave)
struct Work {
  int tile, ks, S, item;  // item: index of the split item (-1: a whole tile)
  int fix_mi;             // fixup pass: the 16-row block this workgroup finishes
  int k_begin, k_end;
  bool ok;
  TileInfo ti;
};

// One pass over the offsets (4 experts per lane, as in locate_tile): the
// per-expert tile counts, their wave prefix sum (the total and each
// expert's first tile), the split, this block's work item and its tile.
// WIDE_OK: the enumeration may form wide items (when p.wide_rem is set);
// without it their code is left out (it runs in every tile's prologue).
template <bool WIDE_OK>
__device__ __forceinline__ Work assign_work(const GemmArgs& p, int b, int pbk) {
  const int lane = threadIdx.x & 63;
  int cnt_tiles[4], mt[4], offe[4], rows_e[4];
  bool wide_e[4];
  int lane_sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane * 4 + u;
    int m = 0, o = 0, c = 0;
    if (e < p.E) {
      o = p.offsets[e];
      c = p.offsets[e + 1] - o;
      m = cdiv(c, BM);
    }
    mt[u] = m;
    offe[u] = o;
    rows_e[u] = c;
    // an expert walked in one pass whose last rows fill at most half a tile:
    // floor(c / BM) full tiles per N panel, and its last rows as one wide
    // item per pair of panels (ceil(tn / 2) of them)
    const int rem = c - (c / BM) * BM;
    wide_e[u] = WIDE_OK && p.wide_rem && rem > 0 && 2 * rem <= BM && m <= p.m_group_min;
    cnt_tiles[u] = wide_e[u] ? (c / BM) * p.tiles_n + (p.tiles_n + 1) / 2 : m * p.tiles_n;
    lane_sum += cnt_tiles[u];
  }
  const int incl = wave_incl_sum(lane_sum);
  const int n_tiles = __builtin_amdgcn_readlane(incl, 63);
  const int C = p.n_cu;
  int tail = n_tiles % C;
  const int nk_all = p.K / pbk;
  // split only where the last round is mostly idle (at most half full) and
  // the launch has at most kSplitMaxRounds rounds; otherwise the
  // fixup pass costs more than the idle compute units.  A split then has
  // S >= 2 parts (C / tail >= 2 and nk_all >= 2), so the tail stays.
  const bool split = p.part != nullptr && tail > 0 && 2 * tail <= C &&
                     n_tiles <= kSplitMaxRounds * C && nk_all >= 2;
  if (!split) tail = 0;
  const int F = n_tiles - tail;
  // the split's part count and K per part; only the split items and the
  // fixup pass use them, so whole tiles skip these divisions
  auto split_parts = [&](int& S, int& kps) {
    S = min(C / tail, nk_all);
    kps = cdiv(nk_all, S) * pbk;
    S = cdiv(p.K, kps);  // parts that are not empty
  };
  Work w{};
  w.S = 1;
  w.ok = false;
  w.item = -1;
  w.ks = 0;
  w.k_begin = 0;
  w.k_end = p.K;
  w.tile = -1;
  w.fix_mi = 0;
  if (p.fixup) {
    if (b < tail * FIXQ) {
      int S, kps;
      split_parts(S, kps);
      w.S = S;
      w.tile = F + b / FIXQ;
      w.item = (b / FIXQ) * S;
      w.fix_mi = b % FIXQ;
    }
  } else {
    const int G = cdiv(F, 8) * 8;
    if (b < G) {
      const int t = (b & 7) * (G / 8) + (b >> 3);
      if (t < F) w.tile = t;
    } else if (tail > 0) {
      int S, kps;
      split_parts(S, kps);
      if (b - G < tail * S) {
        const int j = b - G;
        w.S = S;
        w.tile = F + j / S;
        w.ks = j % S;
        w.item = j;
        w.k_begin = w.ks * kps;
        w.k_end = min(p.K, w.k_begin + kps);
      }
    }
  }
  if (w.tile < 0) return w;
  // the expert holding tile w.tile, from the same prefix sums
  int start = incl - lane_sum;
  int hit_e = -1, hit_start = 0, hit_mt = 0, hit_off = 0, hit_rows = 0, hit_wide = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (w.tile >= start && w.tile < start + cnt_tiles[u]) {
      hit_e = lane * 4 + u;
      hit_start = start;
      hit_mt = mt[u];
      hit_off = offe[u];
      hit_rows = rows_e[u];
      hit_wide = wide_e[u] ? 1 : 0;
    }
    start += cnt_tiles[u];
  }
  const uint64_t hit = __ballot(hit_e >= 0);
  if (hit == 0) return w;
  const int src = __ffsll((unsigned long long)hit) - 1;  // uniform: read from that lane
  TileInfo& ti = w.ti;
  ti.e = __builtin_amdgcn_readlane(hit_e, src);
  const int tstart = __builtin_amdgcn_readlane(hit_start, src);
  const int tmt = __builtin_amdgcn_readlane(hit_mt, src);
  const int toff = __builtin_amdgcn_readlane(hit_off, src);
  // the expert's row count comes from the lane that holds it, not from a
  // second, dependent read of the offsets
  const int c_e = __builtin_amdgcn_readlane(hit_rows, src);
  const int local = w.tile - tstart;
  ti.wide = false;
  if (WIDE_OK && __builtin_amdgcn_readlane(hit_wide, src)) {
    // items per pair of N panels (2j, 2j + 1): the mf full M tiles of panel
    // 2j, those of panel 2j + 1, then the wide item of the last rows (a last
    // odd panel: its mf tiles, then a wide item with no second panel)
    const int mf = c_e / BM;
    const int per = 2 * mf + 1;
    const int j = local / per, r = local - j * per;
    if (r < mf || (r < 2 * mf && 2 * j + 1 < p.tiles_n)) {
      const int second = r >= mf ? 1 : 0;
      ti.n_t = 2 * j + second;
      ti.m_t = r - second * mf;
      ti.nb = BM / 16;
      ti.row0 = toff + BM * ti.m_t;
      ti.row_end = ti.row0 + BM;
    } else {
      ti.wide = true;
      ti.n_t = 2 * j;
      ti.m_t = mf;
      ti.row0 = toff + BM * mf;
      ti.row_end = toff + c_e;
      ti.nb = cdiv(ti.row_end - ti.row0, 16);
    }
    ti.ok = true;
    w.ok = true;
    return w;
  }
  // A large expert's M tiles are walked in ng balanced groups of at most
  // m_group tiles (the first tmt % ng groups hold one tile more); a group
  // covers all N panels, M fastest inside each panel, before the next, so
  // its token rows (the A operand) are reused by every panel while they
  // still sit in the last-level cache.  A small expert is one group.
  const int tn = p.tiles_n;
  if (tmt <= p.m_group_min) {
    // one group (every expert of moderate size): M fastest inside each panel
    ti.n_t = local / tmt;
    ti.m_t = local - ti.n_t * tmt;
  } else {
    const int ng = cdiv(tmt, p.m_group);
    const int g_lo = tmt / ng, g_rem = tmt - g_lo * ng;  // group sizes g_lo + 1 (g_rem of them), g_lo
    const int big = g_rem * (g_lo + 1) * tn;            // tiles in the larger groups
    int q, m0, mq;
    if (local < big) {
      q = local / ((g_lo + 1) * tn);
      m0 = q * (g_lo + 1);
      mq = g_lo + 1;
    } else {
      q = g_rem + (local - big) / (g_lo * tn);
      m0 = g_rem * (g_lo + 1) + (q - g_rem) * g_lo;
      mq = g_lo;
    }
    const int r = local - m0 * tn;
    ti.n_t = r / mq;
    ti.m_t = m0 + (r - ti.n_t * mq);
  }
  // Balanced M tiles: the expert's c rows form nbe = ceil(c / 16) blocks of
  // 16, dealt to its tmt = ceil(c / BM) tiles as evenly as possible (the
  // first nbe % tmt tiles take one block more; every tile takes between 1
  // and BM / 16).  Against full tiles plus one ragged last tile, this
  // removes all padding but the last block's, and the tiles of an (expert,
  // N panel), which run side by side and share the panel, take equal time.
  const int nbe = cdiv(c_e, 16);
  const int b_lo = nbe / tmt, b_rem = nbe - b_lo * tmt;
  const int b0 = ti.m_t * b_lo + min(ti.m_t, b_rem);
  const int b1 = b0 + b_lo + (ti.m_t < b_rem ? 1 : 0);
  ti.nb = b1 - b0;
  ti.row0 = toff + 16 * b0;
  ti.row_end = min(toff + 16 * b1, toff + c_e);
  ti.ok = true;
  w.ok = true;
  return w;
}

// One work item of the ping-pong kernel.  FIX = false: the main pass; FIX =
// true: the fixup pass of the tail split (no K loop: the accumulators are the
// sum of the split items' partials).  WIDE = false: a tile of up to 256 rows
// x one N panel, group X on its first ceil(nb / 2) 16-row blocks, group Y on
// the rest.  WIDE = true: a wide item, up to 128 rows x two N panels, both
// groups on the same rows, X on panel n_t and Y on panel n_t + 1; its stage
// is an A slot of 128 rows (16 KiB) and a B slot of both panels (64 KiB),
// rings of 2 (160 KiB); X issues the A loads and its panel's B loads, Y its
// panel's B loads.  A separate instantiation, so that the whole tiles' loop
// carries no test for it.
template <bool UP, int PBK, bool FIX, bool WIDE>
__device__ __forceinline__ void pp_tile(const GemmArgs p, const Work wk, char* lds) {
  using namespace pp;
  using C = Cfg<PBK>;
  constexpr int SLOT = C::SLOT, HALF = C::HALF, KS = C::KS, LD = C::LD;
  constexpr int RA = WIDE ? 2 : C::RA, RB = WIDE ? 2 : C::RB;
  constexpr int SLOT_A = WIDE ? SLOT / 2 : SLOT;  // A stage: 128 or 256 rows
  constexpr int SLOT_B = WIDE ? 2 * SLOT : SLOT;  // B stage: two panels or one
  constexpr int B_RING = RA * SLOT_A;             // B slots start after the A slots
  static_assert(RA * SLOT_A + RB * SLOT_B <= C::LDS_BYTES, "LDS");
  constexpr int LDA = WIDE ? LD / 2 : LD;         // A loads per X wave per stage
  const TileInfo& ti0 = wk.ti;
  // the tile is the same for every lane: keep it in scalar registers
  const int t_e = __builtin_amdgcn_readfirstlane(ti0.e);
  const int t_row0 = __builtin_amdgcn_readfirstlane(ti0.row0);
  const int t_row_end = __builtin_amdgcn_readfirstlane(ti0.row_end);
  const int t_n = __builtin_amdgcn_readfirstlane(ti0.n_t);
  // the tile's nb 16-row blocks: the first ceil(nb / 2) go to group X, the
  // rest to group Y; each wave computes only its group's blocks
  const int t_nb = __builtin_amdgcn_readfirstlane(ti0.nb);
  const int t_bx = (t_nb + 1) >> 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool X = wave < 4;       // leading group: LDS rows 0-127, issues the A loads
  const int wg = wave & 3;       // wave inside its group
  const int my_nb = WIDE ? t_nb : (X ? t_bx : t_nb - t_bx);  // blocks this wave computes (0..MI)
  const int grow0 = WIDE ? 0 : (X ? 0 : 16 * t_bx);          // the group's first row inside the tile
  const int grow_end = min(t_row_end, t_row0 + grow0 + 16 * my_nb);  // its row bound
  const int K = p.K, N = p.N;
  // the group's N panel (wide items: Y takes the next one; past the last
  // panel its loads read valid columns and nothing is stored)
  const int n0 = (t_n + (WIDE && !X ? 1 : 0)) * (UP ? 128 : 256);
  const uint32_t lds0 = lds_addr_of(lds);
  const int k_begin = __builtin_amdgcn_readfirstlane(wk.k_begin);
  const int k_end = __builtin_amdgcn_readfirstlane(wk.k_end);
  const int nk = FIX ? 0 : (k_end - k_begin) / PBK;
  const int w_item = __builtin_amdgcn_readfirstlane(wk.item);
  const int w_S = __builtin_amdgcn_readfirstlane(wk.S);
  const int w_fix_mi = __builtin_amdgcn_readfirstlane(wk.fix_mi);

  // ---- loads.  X: load j = LD wg + q fills A rows RPL j .. RPL (j + 1) - 1;
  // lane l reads 16 B of row RPL j + l / CPR (chunk swizzled by the row).
  // Y: load j = LD wg + q fills K rows 4 (j % (PBK / 4)) .. + 3 of B half
  // j / (PBK / 4) = wg / 2; lane l reads 16 B of row 4 (j % (PBK / 4)) + l / 16.
  // Its lane part depends on q % 4 only (q / 4 adds 16 rows).
  uint32_t ld_off[LD];  // X: A byte offsets at k_begin; Y: B byte offsets (q < 4)
  const char* ld_base0; // stage-0 scalar base
  const int b_half = wg >> 1;
  // B offsets of the group's panel (whole tiles: group Y's loads)
  auto b_offsets = [&]() {
    const bf16_t* b_mat = UP ? (b_half ? p.B1 : p.B0) : p.B0;
    const int n0h = UP ? n0 : n0 + b_half * 128;
#pragma unroll
    for (int u = 0; u < LD; ++u) {
      const int krow = 4 * (u & 3) + (lane >> 4);  // row inside its 16-row group
      const int chunk = (lane & 15) ^ b_swz<128>(krow);
      int col = n0h + chunk * 8;
      if (col >= N) col = N - 8;  // padding columns read valid data; results are discarded
      ld_off[u] = ((uint32_t)krow * (uint32_t)N + (uint32_t)col) * 2u;
    }
    ld_base0 = uniform_ptr(b_mat + (size_t)t_e * K * N +
                           (size_t)(k_begin + (PBK / 2) * (wg & 1)) * N);
  };
  // A offsets (X): load j = LDA wg + q fills LDS rows RPL j .. RPL (j + 1) - 1
  auto a_offset = [&](int q) {
    const int row = (wg * LDA + q) * C::RPL + lane / C::CPR;  // LDS row
    const int chunk = (lane % C::CPR) ^ a_swz16<PBK>(row);
    // LDS rows 0-127 hold group X's blocks, 128-255 group Y's (wide items:
    // rows 0-127 only, the blocks of both)
    const int j = row & 127;
    const int gnb = WIDE ? t_nb : (row < 128 ? t_bx : t_nb - t_bx);
    int r = t_row0 + ((WIDE || row < 128) ? 0 : 16 * t_bx) + j;
    // rows past the group's blocks or the expert's rows read a valid row;
    // their results are never stored
    if (j >= 16 * gnb || r >= t_row_end) r = t_row0;
    const int src_row = p.gather ? p.gather[r] : r;
    return ((uint32_t)src_row * (uint32_t)K + (uint32_t)(k_begin + chunk * 8)) * 2u;
  };
  uint32_t a_off[LDA];  // wide items: X's A byte offsets (its ld_off are B's)
  const char* a_base0 = nullptr;
  if constexpr (!WIDE) {
    if (X) {
#pragma unroll
      for (int q = 0; q < LD; ++q) ld_off[q] = a_offset(q);
      ld_base0 = uniform_ptr(p.A);
    } else {
      b_offsets();
    }
  } else {
    if (X) {
#pragma unroll
      for (int q = 0; q < LDA; ++q) a_off[q] = a_offset(q);
      a_base0 = uniform_ptr(p.A);
    }
    b_offsets();
  }
  auto issue_a = [&](int kt, int slot, int q) {
    const uint32_t dst = lds0 + (uint32_t)(slot * SLOT_A + (wg * LDA + q) * 1024);
    if constexpr (WIDE) lds_dma16_s(a_off[q], a_base0 + (size_t)kt * PBK * 2, dst);
    else lds_dma16_s(ld_off[q], ld_base0 + (size_t)kt * PBK * 2, dst);
  };
  // wide items: the group's panel is the first or the second half of the B slot
  const int b_panel = (WIDE && !X) ? SLOT : 0;
  auto issue_b = [&](int kt, int slot, int q) {
    const uint32_t dst = lds0 + (uint32_t)(B_RING + slot * SLOT_B + b_panel + (wg * LD + q) * 1024);
    const char* base = ld_base0 + ((size_t)kt * PBK + (size_t)(16 * (q >> 2))) * N * 2;
    lds_dma16_s(ld_off[q], uniform_ptr(base), dst);
  };

  // ---- fragment read offsets (bytes inside a stage slot)
  const int l15 = lane & 15, g = lane >> 4;
  const int wrow0 = (WIDE || X) ? 0 : 128;
  const int a_s = a_swz16<PBK>(l15);
  const int a_rd0 = (wrow0 + l15) * (PBK * 2) + ((g ^ a_s) << 4);        // K step 0
  const int a_rd1 = (wrow0 + l15) * (PBK * 2) + (((g + 4) ^ a_s) << 4);  // K step 1 (PBK = 64)
  // B: blocks nj = 0, 1 in half 0, nj = 2, 3 the same columns of half 1; K
  // step 1 adds 32 rows (8 KiB, same swizzle)
  int b_rd[2], b_rd4[2];
  const int b_kr = g * 8 + (l15 >> 2);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    b_rd[c] = b_off<128>(b_kr, wg * 32 + c * 16 + (lane & 3) * 4);
    b_rd4[c] = b_off<128>(b_kr + 4, wg * 32 + c * 16 + (lane & 3) * 4);
  }

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 fa[KS][MI], fb[KS][NJ];  // fragments of one stage: [K step][block]
  // memory phase: read the stage's fragments (A slot sa, B slot sb), issue
  // this wave's loads of stage ld_kt into slot ld_slot, wait for the reads
  auto memory = [&](int sa, int sb, int ld_kt, int ld_slot) {
    const char* As = lds + sa * SLOT_A;
    const char* Bs = lds + B_RING + sb * SLOT_B + b_panel;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj) {
        const char* Bh = Bs + (nj >> 1) * HALF + ks * 8192;
        const bf16x4 lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Bh + b_rd[nj & 1]));
        const bf16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Bh + b_rd4[nj & 1]));
        fb[ks][nj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      const char* Ak = As + (ks ? a_rd1 : a_rd0);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        if (mi < my_nb) fa[ks][mi] = *reinterpret_cast<const bf16x8*>(Ak + mi * 16 * PBK * 2);
      // the loads after the reads of each K step (half of them each when
      // there are two)
      if (ld_kt < nk) {
        if constexpr (WIDE) {
          if (X) {
#pragma unroll
            for (int q = ks * (LDA / KS); q < (ks + 1) * (LDA / KS); ++q) issue_a(ld_kt, ld_slot, q);
          }
#pragma unroll
          for (int q = ks * (LD / KS); q < (ks + 1) * (LD / KS); ++q) issue_b(ld_kt, ld_slot, q);
        } else {
#pragma unroll
          for (int q = ks * (LD / KS); q < (ks + 1) * (LD / KS); ++q) {
            if (X) issue_a(ld_kt, ld_slot, q);
            else issue_b(ld_kt, ld_slot, q);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  };
  auto compute = [&]() {
    __builtin_amdgcn_s_setprio(1);
    // blocks in (16-row block, K step) order: one test per block of a
    // partial tile
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

  // The two groups run separate loops with the same barrier count: one
  // after the prologue and two per stage.  Slots rotate: stage s sits in A
  // slot s % RA and B slot s % RB.
  if (FIX) {
    // no K loop
  } else if (X) {
    // prologue: A(0) .. A(RA - 2) (wide items: with the panel's B); wait for A(0)
    for (int s = 0; s < RA - 1 && s < nk; ++s) {
#pragma unroll
      for (int q = 0; q < LDA; ++q) issue_a(s, s, q);
      if (WIDE) {
#pragma unroll
        for (int q = 0; q < LD; ++q) issue_b(s, s, q);
      }
    }
    if (WIDE) wait_vmcnt<0>();  // rings of 2: stage 0 is everything issued
    else wait_groups<LD>(min(RA - 2, nk - 1));
    __builtin_amdgcn_s_barrier();
    int sa = 0, sb = 0;
    for (int s = 0; s < nk; ++s) {
      const int la = sa == 0 ? RA - 1 : sa - 1;  // slot of stage s - 1 = of s + RA - 1
      memory(sa, sb, s + RA - 1, la);            // phase 2s
      __builtin_amdgcn_s_barrier();
      compute();                                  // phase 2s + 1
      // A(s + 1) has landed once the later stages' loads are all that remain
      // (wide items: with the panel's B(s + 1), everything outstanding)
      if (WIDE) wait_vmcnt<0>();
      else wait_groups<LD>(min(RA - 2, nk - 2 - s));
      __builtin_amdgcn_s_barrier();
      sa = sa == RA - 1 ? 0 : sa + 1;
      sb = sb == RB - 1 ? 0 : sb + 1;
    }
  } else {
    // prologue: B(0) .. B(RB - 2); wait for B(0)
    for (int s = 0; s < RB - 1 && s < nk; ++s)
#pragma unroll
      for (int q = 0; q < LD; ++q) issue_b(s, s, q);
    if (WIDE) wait_vmcnt<0>();
    else wait_groups<LD>(min(RB - 2, nk - 1));
    __builtin_amdgcn_s_barrier();
    int sa = 0, sb = 0;
    for (int s = 0; s < nk; ++s) {
      if (s > 0) {
        compute();  // phase 2s: stage s - 1
        // wide items: only this group reads its panel, and it reads B(s) in
        // phase 2s + 1: its loads (issued in phase 2s - 1) are awaited here
        if (WIDE) wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();
      // phase 2s + 1: read stage s, load B(s + RB - 1) into the slot of stage
      // s - 1; then (whole tiles: X reads B(s + 1) next phase) B(s + 1) must
      // have landed
      const int lb = sb == 0 ? RB - 1 : sb - 1;
      memory(sa, sb, s + RB - 1, lb);
      if (!WIDE) wait_groups<LD>(min(RB - 2, nk - 2 - s));
      __builtin_amdgcn_s_barrier();
      sa = sa == RA - 1 ? 0 : sa + 1;
      sb = sb == RB - 1 ? 0 : sb + 1;
    }
    if (nk > 0) compute();  // phase 2 nk: stage nk - 1 (LDS is free: all reads and loads waited for)
  }

  // partial accumulators of split item i: [i][wave][mi * NJ + nj][lane] x 4 floats
  f32x4* part_base = reinterpret_cast<f32x4*>(p.part) + (size_t)(w_item < 0 ? 0 : w_item) * 512 * MI * NJ;
  if (FIX) {
    // sum the S partials of this tail tile in part order
    // (this workgroup's 16-row block fix_mi of every wave only, held in
    // acc[0]; the epilogue places it at block fix_mi)
    const int S = w_S;
    for (int sp = 0; sp < S; ++sp) {
      const f32x4* src = part_base + (size_t)sp * 512 * MI * NJ;
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj)
        acc[0][nj] += src[((size_t)wave * MI * NJ + w_fix_mi * NJ + nj) * 64 + lane];
    }
  } else if (w_item >= 0) {
    // a split item: store the partial accumulators; the fixup pass finishes the tile
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < NJ; ++nj)
        part_base[((size_t)wave * MI * NJ + mi * NJ + nj) * 64 + lane] = acc[mi][nj];
    return;
  }

  // ---- epilogue (accumulator layout of a 16 x 16 block: column lane % 16,
  // rows 4 * (lane / 16) + i), staged through the wave's own LDS area
  const int col_l = lane & 15;
  const int row_l = (lane >> 4) * 4;
  // the fixup pass finishes one block per wave (acc[0] = block fix_mi)
  constexpr int EMI = FIX ? 1 : MI;
  const int mi_off = FIX ? w_fix_mi : 0;
  if (UP) {
    constexpr int OC = 32, SS = OC + 8;  // output columns per wave; staging stride (bf16)
    bf16_t* sb = reinterpret_cast<bf16_t*>(lds + wave * 16 * SS * 2);
    const int ocol0 = n0 + wg * OC;
    const int nout = p.h_out ? 3 : 1;  // SiLU(h) u, then (training) h and u
#pragma unroll
    for (int mi = 0; mi < EMI; ++mi) {
      if (mi + mi_off >= my_nb) break;
      for (int o = 0; o < nout; ++o) {
        bf16_t* dst = o == 0 ? p.a_out : (o == 1 ? p.h_out : p.u_out);
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float h = acc[mi][nj][i], u = acc[mi][nj + 2][i];
            sb[(row_l + i) * SS + nj * 16 + col_l] = f32_to_bf16(o == 0 ? silu(h) * u : (o == 1 ? h : u));
          }
        // 16 rows x 4 chunks of 16 B: one per lane
        const int r = lane >> 2, c = lane & 3;
        const int row = t_row0 + grow0 + (mi + mi_off) * 16 + r;
        const int col = ocol0 + c * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(sb + r * SS + c * 8);
        if (row < grow_end && col < N)
          *reinterpret_cast<u32x4*>(dst + (size_t)row * N + col) = v;
      }
    }
  } else {
    // the wave's columns: n0 + h * 128 + wg * 32 + [0, 32) for halves h = 0, 1
    if (p.y_h) {
      // compact rows: each 16-row block is staged, then every lane reads the
      // 8 columns of its two row segments (4 LDS reads, one wait), scales,
      // converts and stores them; the non-temporal choice is made once
      auto compact = [&](auto nt_tag) {
        constexpr bool NT = decltype(nt_tag)::value;
        constexpr int SS = 64 + 4;  // staging stride in floats
        float* sf = reinterpret_cast<float*>(lds + wave * 16 * SS * 4);
        const int segs = N >> 5;
#pragma unroll
        for (int mi = 0; mi < EMI; ++mi) {
          if (mi + mi_off >= my_nb) break;
#pragma unroll
          for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
            for (int i = 0; i < 4; ++i) sf[(row_l + i) * SS + nj * 16 + col_l] = acc[mi][nj][i];
          f32x4 va[2], vb[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int idx = q * 64 + lane;
            const float* src = sf + (idx >> 3) * SS + (idx & 7) * 8;
            va[q] = *reinterpret_cast<const f32x4*>(src);
            vb[q] = *reinterpret_cast<const f32x4*>(src + 4);
          }
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int idx = q * 64 + lane;
            const int r = idx >> 3, c = idx & 7;
            const int row = t_row0 + grow0 + (mi + mi_off) * 16 + r;
            const int col = n0 + (c >> 2) * 128 + wg * 32 + (c & 3) * 8;
            store_seg_f16v<NT>(va[q], vb[q], p.y_h + (size_t)row * N + col,
                               p.y_s + (size_t)row * segs + (col >> 5),
                               row < grow_end && col < N, (c & 3) == 0);
          }
        }
      };
      if (p.nt_y) compact(std::true_type{});
      else compact(std::false_type{});
    } else if (p.y_perm) {
      constexpr int SS = 64 + 4;  // staging stride in floats
      float* sf = reinterpret_cast<float*>(lds + wave * 16 * SS * 4);
#pragma unroll
      for (int mi = 0; mi < EMI; ++mi) {
        if (mi + mi_off >= my_nb) break;
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj)
#pragma unroll
          for (int i = 0; i < 4; ++i) sf[(row_l + i) * SS + nj * 16 + col_l] = acc[mi][nj][i];
        // 16 rows x 16 chunks of 16 B; two separate loops, so that the
        // compiler keeps the non-temporal hint (merging the two stores drops it)
        if (p.nt_y) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int idx = q * 64 + lane;
            const int r = idx >> 4, c = idx & 15;
            const int row = t_row0 + grow0 + (mi + mi_off) * 16 + r;
            const int col = n0 + (c >> 3) * 128 + wg * 32 + (c & 7) * 4;
            const f32x4 v = *reinterpret_cast<const f32x4*>(sf + r * SS + c * 4);
            if (row < grow_end && col < N)
              __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p.y_perm + (size_t)row * N + col));
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int idx = q * 64 + lane;
            const int r = idx >> 4, c = idx & 15;
            const int row = t_row0 + grow0 + (mi + mi_off) * 16 + r;
            const int col = n0 + (c >> 3) * 128 + wg * 32 + (c & 7) * 4;
            const f32x4 v = *reinterpret_cast<const f32x4*>(sf + r * SS + c * 4);
            if (row < grow_end && col < N)
              *reinterpret_cast<f32x4*>(p.y_perm + (size_t)row * N + col) = v;
          }
        }
      }
    }
    if (p.y) {
#pragma unroll
      for (int mi = 0; mi < EMI; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = t_row0 + grow0 + (mi + mi_off) * 16 + row_l + i;
          if (row >= grow_end) continue;
          const int tgt = p.scatter ? p.scatter[row] : row;
          float* yrow = p.y + (size_t)tgt * N;
          const float wgt = p.row_w ? p.row_w[row] : 1.f;
#pragma unroll
          for (int nj = 0; nj < NJ; ++nj) {
            const int col = n0 + (nj >> 1) * 128 + wg * 32 + (nj & 1) * 16 + col_l;
            if (col < N) unsafeAtomicAdd(yrow + col, wgt * acc[mi][nj][i]);
          }
        }
      }
    }
  }
}

// FIX = false: the main pass; FIX = true: the fixup pass of the tail split.
// WIDE_OK: the launch may hold wide items (p.wide_rem = 1); without them the
// kernel holds no wide-item code at all (its presence alone changes the
// register assignment of the whole tiles' code: 0.5-0.8% on a short K loop).
template <bool UP, int PBK, bool FIX, bool WIDE_OK>
__global__ __launch_bounds__(512, 1) void grouped_gemm_bf16_pp_kernel(GemmArgs p) {
  using C = pp::Cfg<PBK>;
  // the fixup pass uses LDS only for the epilogue's per-wave staging (at
  // most 16 rows x 68 floats per wave): sized so that several of its short
  // workgroups share a compute unit
  constexpr int FIX_LDS = pp::NW * 16 * 68 * 4;
  __shared__ __attribute__((aligned(1024))) char lds[FIX ? FIX_LDS : C::LDS_BYTES];
  const Work wk = assign_work<WIDE_OK>(p, blockIdx.x, PBK);
  if (!wk.ok) return;
  if constexpr (WIDE_OK) {
    if (wk.ti.wide) {
      pp_tile<UP, PBK, FIX, true>(p, wk, lds);
      return;
    }
  }
  pp_tile<UP, PBK, FIX, false>(p, wk, lds);
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
                              float* __restrict__ a_out, float* __restrict__ h_out,
                              float* __restrict__ u_out) {
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
  if (h_out) {
    h_out[i] = h;
    u_out[i] = v;
  }
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

// the general kernel's wave grid (2 x 4 waves) and accumulator columns per tile
constexpr int UP_WN = 4, UP_BNA = 256, DN_WN = 4, DN_BNA = 256;
// An expert whose A rows exceed kMGroupMinMB is walked in passes of at most
// kMGroupMB of A rows, each pass covering all N panels (its rows are then
// re-read from the last-level cache, not HBM)
constexpr long long kMGroupMB = 32, kMGroupMinMB = 64;
// Wide items (see assign_work) from this K on
constexpr int kWideMinK = 2048;

int num_cus() {
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

// Workspace of the ping-pong kernel's tail split: one 256 x 256 fp32
// partial tile per split item, at most one item per compute unit.
size_t pp_part_bytes(int n_cu) { return (size_t)n_cu * BM * 256 * sizeof(float); }

// a_rows_bytes: size of the A matrix the kernel may read (rows that can be
// addressed times K times 2 bytes); p.part: the caller's workspace
// (ws_bytes bytes), used when large enough
template <bool UP, int WM, int WN, int BNA>
hipError_t launch_gemm(GemmArgs& p, int rows, int E, int ncols, unsigned long long a_rows_bytes,
                       size_t ws_bytes, hipStream_t s) {
  static_assert(BNA == 256, "ping-pong kernel tile width");
  p.tiles_n = cdiv(ncols, UP ? BNA / 2 : BNA);
  {
    const long long a_tile = (long long)BM * p.K * 2;
    p.m_group = (int)std::max(1LL, (kMGroupMB << 20) / a_tile);
    p.m_group_min = (int)std::max(1LL, (kMGroupMinMB << 20) / a_tile);
  }
  const long long tiles = (long long)max_tiles_m(rows, E) * p.tiles_n;
  const long long grid = (tiles + 7) / 8 * 8;
  p.grid_per_xcd = (int)(grid / 8);
  if (p.K % 64 == 0 && a_rows_bytes < (1ull << 32)) {
    // main pass: the whole tiles plus at most n_cu split items; then the
    // fixup pass over at most n_cu / 2 tail tiles (both derive the split
    // from the device offsets; without a workspace there is none)
    p.n_cu = num_cus();
    p.fixup = 0;
    // wide items where the K loop is long enough to carry their rings of
    // two (measured: with K = 1408, 22 stages, they cost 2.4%)
    p.wide_rem = p.K >= kWideMinK ? 1 : 0;
    // a y_perm beyond the 256 MB last-level cache is streamed past it (the
    // combine re-reads it from HBM either way); a smaller one stays cached
    // for the combine (DeepSeek shape, 1.6 GB: +2%; Mixtral, 134 MB: cached)
    p.nt_y = (p.y_perm && (unsigned long long)rows * ncols * 4 > (256ull << 20)) ||
             (p.y_h && (unsigned long long)rows * ncols * 2 > (256ull << 20));
    if (ws_bytes < pp_part_bytes(p.n_cu)) p.part = nullptr;
    const long long grid_pp = grid + (p.part ? p.n_cu : 0);
    // both passes derive the same items, so they take the same instantiation
    auto launch = [&](auto wide_ok) {
      constexpr bool W = decltype(wide_ok)::value;
      hipLaunchKernelGGL((grouped_gemm_bf16_pp_kernel<UP, 64, false, W>),
                         dim3((unsigned)grid_pp), dim3(64 * pp::NW), 0, s, p);
      if (p.part) {
        p.fixup = 1;
        hipLaunchKernelGGL((grouped_gemm_bf16_pp_kernel<UP, 64, true, W>),
                           dim3((unsigned)(p.n_cu / 2 * FIXQ)), dim3(64 * pp::NW), 0, s, p);
      }
    };
    if (p.wide_rem) launch(std::true_type{});
    else launch(std::false_type{});
    return hipGetLastError();
  }
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<UP, WM, WN, BNA>), dim3((unsigned)grid),
                     dim3(64 * WM * WN), 0, s, p);
  return hipGetLastError();
}

}  // namespace

size_t ffn_workspace_bytes(int E, int rows, int d, int f) {
  (void)E; (void)rows; (void)d; (void)f;
  return pp_part_bytes(num_cus());
}

hipError_t launch_expert_up(const void* x, const int32_t* gather_idx, const int32_t* offsets,
                            int E, int rows, int d, int f, bool bf16, const void* W_gate,
                            const void* W_up, void* a_out, void* h_out, void* u_out, void* ws,
                            size_t ws_bytes, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (!bf16) {
    const size_t n = (size_t)rows * f;
    hipLaunchKernelGGL(up_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(x), gather_idx, offsets, E, rows, d, f,
                       static_cast<const float*>(W_gate), static_cast<const float*>(W_up),
                       static_cast<float*>(a_out), static_cast<float*>(h_out),
                       static_cast<float*>(u_out));
    return hipGetLastError();
  }
  GemmArgs p{};
  p.A = static_cast<const bf16_t*>(x);
  p.h_out = static_cast<bf16_t*>(h_out);
  p.u_out = static_cast<bf16_t*>(u_out);
  p.gather = gather_idx;
  p.offsets = offsets;
  p.E = E; p.rows = rows; p.K = d; p.N = f;
  p.B0 = static_cast<const bf16_t*>(W_gate);
  p.B1 = static_cast<const bf16_t*>(W_up);
  p.a_out = static_cast<bf16_t*>(a_out);
  p.part = static_cast<float*>(ws);
  // gather entries are < rows (documented), so A spans at most rows x d
  return launch_gemm<true, 2, UP_WN, UP_BNA>(p, rows, E, f, (unsigned long long)rows * d * 2,
                                             ws ? ws_bytes : 0, s);
}

hipError_t launch_expert_down(const void* a, const int32_t* offsets, int E, int rows, int f,
                              int d, bool bf16, const void* W_down, float* y_perm,
                              const int32_t* scatter_idx, const float* row_w, float* y, void* ws,
                              size_t ws_bytes, hipStream_t s) {
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
  p.part = static_cast<float*>(ws);
  return launch_gemm<false, 2, DN_WN, DN_BNA>(p, rows, E, d, (unsigned long long)rows * f * 2,
                                              ws ? ws_bytes : 0, s);
}

hipError_t launch_expert_down_f16(const void* a, const int32_t* offsets, int E, int rows, int f,
                                  int d, const void* W_down, uint16_t* y_h, float* y_s, void* ws,
                                  size_t ws_bytes, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  GemmArgs p{};
  p.A = static_cast<const bf16_t*>(a);
  p.offsets = offsets;
  p.E = E; p.rows = rows; p.K = f; p.N = d;
  p.B0 = static_cast<const bf16_t*>(W_down);
  p.y_h = y_h;
  p.y_s = y_s;
  p.part = static_cast<float*>(ws);
  return launch_gemm<false, 2, DN_WN, DN_BNA>(p, rows, E, d, (unsigned long long)rows * f * 2,
                                              ws ? ws_bytes : 0, s);
}

}  // namespace moe
