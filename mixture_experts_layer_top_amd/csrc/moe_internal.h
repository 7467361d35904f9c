// Internal declarations shared by the HIP translation units of libmoe.so:
// device helpers (bf16 conversion, wave reductions) and the host-side
// launchers each kernel file exports to the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float -> bfloat16 with round-to-nearest-even: gfx950's conversion
// instruction (v_cvt_pk_bf16_f32, two values per instruction; NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// SiLU(h) = h / (1 + exp(-h)), with the hardware reciprocal (about 1 ulp)
__device__ __forceinline__ float silu(float h) {
  return h * __builtin_amdgcn_rcpf(1.0f + __expf(-h));
}

// Inclusive prefix sum over the wave's 64 lanes (every lane active): a
// Hillis-Steele scan inside each row of 16 lanes by DPP row shifts (lanes
// shifted in from outside the row read 0), then the totals of the rows
// below, read from lanes 15, 31 and 47, added to each row.  The shuffles
// this replaces each took a round trip through the LDS permute unit, in a
// dependent chain (at the head of every GEMM tile, for one).
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Round up a / b.
__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// ------------------------------------------------------------------------
// host launchers (each returns a hipError_t of the launch)
// ------------------------------------------------------------------------

int device_cu_count();  // compute units of the current device

hipError_t launch_route(const void* x, const void* W_r, const float* bias, int T, int d, int E,
                        int k, bool renorm, bool bf16, int32_t* idx, float* w, float* logits_out,
                        hipStream_t s);

size_t permute_workspace_bytes(int T, int E, int k);
// allocation-free permute: the static device scratch of this many bytes and
// its address on the current device (looked up once per device)
constexpr size_t kNoAllocScratchBytes = 1u << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_permute(const int32_t* idx, const float* topk_w, const void* x, int T, int d,
                          int E, int k, bool bf16, int32_t* counts, int32_t* offsets,
                          int32_t* perm_token, int32_t* inv, float* perm_w, void* x_perm,
                          void* ws, hipStream_t s);

size_t ffn_workspace_bytes(int E, int rows, int d, int f);
hipError_t launch_expert_up(const void* x, const int32_t* gather_idx, const int32_t* offsets,
                            int E, int rows, int d, int f, bool bf16, const void* W_gate,
                            const void* W_up, void* a_out, void* h_out, void* u_out, void* ws,
                            size_t ws_bytes, hipStream_t s);
hipError_t launch_expert_down(const void* a, const int32_t* offsets, int E, int rows, int f,
                              int d, bool bf16, const void* W_down, float* y_perm,
                              const int32_t* scatter_idx, const float* row_w, float* y, void* ws,
                              size_t ws_bytes, hipStream_t s);
// layer 1 (bf16) with the compact output: fp16 y_h [rows, d] and one
// restoring factor per 32-column row segment, y_s [rows, d / 32] (d % 32 == 0)
hipError_t launch_expert_down_f16(const void* a, const int32_t* offsets, int E, int rows, int f,
                                  int d, const void* W_down, uint16_t* y_h, float* y_s, void* ws,
                                  size_t ws_bytes, hipStream_t s);

hipError_t launch_combine(const float* y_perm, const int32_t* inv, const float* topk_w, int T,
                          int d, int k, const float* y_shared, const float* gate_logit,
                          bool accumulate, float* y, hipStream_t s);
// the combine over compact rows (y_h, y_s as written by launch_expert_down_f16;
// the shared term in the same form, ys_h [T, d], ys_s [T, d / 32], or NULL)
hipError_t launch_combine_f16(const uint16_t* y_h, const float* y_s, const int32_t* inv,
                              const float* topk_w, int T, int d, int k, const uint16_t* ys_h,
                              const float* ys_s, const float* gate_logit, bool accumulate,
                              float* y, hipStream_t s);

hipError_t launch_probe_mfma(int blocks, int iters, const void* ops, uint64_t* ticks,
                             hipStream_t s);
hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);

// backward
// the same over compact rows (y_h, y_s and the shared ys_h, ys_s as written
// by launch_expert_down_f16)
hipError_t launch_combine_backward_f16(const float* dy, const uint16_t* y_h, const float* y_s,
                                       const int32_t* inv, const float* topk_w, int T, int d,
                                       int k, bool bf16, const uint16_t* ys_h, const float* ys_s,
                                       const float* gate_logit, void* dy_perm, float* dw,
                                       void* dy_shared, float* dgate, hipStream_t s);
hipError_t launch_combine_backward(const float* dy, const float* y_perm, const int32_t* inv,
                                   const float* topk_w, int T, int d, int k, bool bf16,
                                   const float* y_shared, const float* gate_logit, void* dy_perm,
                                   float* dw, void* dy_shared, float* dgate, hipStream_t s);
size_t ffn_backward_workspace_bytes(int E, int rows, int d, int f);
hipError_t launch_expert_down_backward(const void* dy_perm, const int32_t* offsets, int E,
                                       int rows, int f, int d, bool bf16, const void* W_down,
                                       const void* h, const void* u, const void* act,
                                       void* dhu, float* dW_down, void* ws, size_t ws_bytes,
                                       hipStream_t s);
hipError_t launch_expert_up_backward(const void* x, const int32_t* gather_idx,
                                     const int32_t* offsets, int E, int rows, int d, int f,
                                     bool bf16, const void* W_gate, const void* W_up,
                                     const void* dhu, float* dx_perm, int accumulate,
                                     float* dW_gate, float* dW_up, void* ws, size_t ws_bytes,
                                     hipStream_t s);
hipError_t launch_unpermute(const float* dx_perm, const int32_t* inv, int T, int d, int k,
                            bool accumulate, float* dx, hipStream_t s);
hipError_t launch_topk_weights_backward(const float* logits, const int32_t* idx, const float* dw,
                                        int T, int E, int k, bool renorm, float* dL,
                                        hipStream_t s);
size_t linear_backward_workspace_bytes(int T, int d, int E);
hipError_t launch_linear_backward(const void* x, const void* W, const float* G, int T, int d,
                                  int E, bool bf16, float* dW, float* db, float* dx, void* ws,
                                  hipStream_t s);

}  // namespace moe
