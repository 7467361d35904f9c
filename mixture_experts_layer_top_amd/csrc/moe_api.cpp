// C ABI of libmoe.so: argument validation on the host, then the launches.
// Every check happens before anything is enqueued, so a rejected call has
// no effect on the stream.  See include/moe.h for the contract of each call.
#include "../../include/moe.h"

#include "moe_internal.h"

#include <algorithm>

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
bool dims_ok(int v) { return v > 0 && (v % 8) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument (null pointer, size out of range, or k > E)";
    case MOE_ERR_UNSUPPORTED:
      return "unsupported argument (misaligned pointer, dimension not a multiple of 8, or unknown enum)";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int moe_route(const void* x, const void* W_r, const float* bias, int T, int d, int E, int k,
              int score, int dtype, int32_t* topk_idx, float* topk_w, float* logits_out,
              hipStream_t stream) {
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E || d <= 0) return MOE_ERR_INVALID;
  if ((long long)T * k >= (1ll << 31) || (long long)T * E >= (1ll << 31)) return MOE_ERR_INVALID;
  if (!dtype_ok(dtype) || (score != MOE_SOFTMAX_TOPK_RENORM && score != MOE_SOFTMAX_TOPK))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !W_r || !topk_idx || !topk_w) return MOE_ERR_INVALID;
  if (d % 8) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(W_r) || !aligned16(topk_idx) || !aligned16(topk_w) ||
      (bias && !aligned16(bias)) || (logits_out && !aligned16(logits_out)))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_route(x, W_r, bias, T, d, E, k, score == MOE_SOFTMAX_TOPK_RENORM,
                                      dtype == MOE_BF16, topk_idx, topk_w, logits_out, stream));
}

size_t moe_permute_workspace_size(int T, int E, int k) {
  if (T < 0 || E < 1 || E > 256 || k < 1) return 0;
  return moe::permute_workspace_bytes(T, E, k);
}

int moe_permute(const int32_t* topk_idx, const float* topk_w, const void* x, int T, int d, int E,
                int k, int dtype, int32_t* counts, int32_t* offsets, int32_t* perm_token,
                int32_t* inv, float* perm_w, void* x_perm, void* workspace, size_t ws_bytes,
                hipStream_t stream) {
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E) return MOE_ERR_INVALID;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_INVALID;
  if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID;
  if (T > 0 && (!topk_idx || !perm_token || !inv)) return MOE_ERR_INVALID;
  if (perm_w && !topk_w) return MOE_ERR_INVALID;
  if (x_perm) {
    if (!x) return MOE_ERR_INVALID;
    if (!dims_ok(d)) return d <= 0 ? MOE_ERR_INVALID : MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_UNSUPPORTED;
  }
  const size_t need = moe::permute_workspace_bytes(T, E, k);
  if (need > 0 && (!workspace || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(counts) || !aligned16(offsets) ||
      !aligned16(perm_token) || !aligned16(inv) || (perm_w && !aligned16(perm_w)))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_permute(topk_idx, topk_w, x, T, d, E, k, dtype == MOE_BF16, counts,
                                        offsets, perm_token, inv, perm_w, x_perm, workspace,
                                        stream));
}

int moe_permute_noalloc(const int32_t* topk_idx, const float* topk_w, const void* x, int T, int d,
                        int E, int k, int dtype, int32_t* counts, int32_t* offsets,
                        int32_t* perm_token, int32_t* inv, float* perm_w, void* x_perm,
                        hipStream_t stream) {
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E) return MOE_ERR_INVALID;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_INVALID;
  if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID;
  if (T > 0 && (!topk_idx || !perm_token || !inv)) return MOE_ERR_INVALID;
  if (perm_w && !topk_w) return MOE_ERR_INVALID;
  if (x_perm) {
    if (!x) return MOE_ERR_INVALID;
    if (!dims_ok(d)) return d <= 0 ? MOE_ERR_INVALID : MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_UNSUPPORTED;
  }
  if (moe::permute_workspace_bytes(T, E, k) > moe::kNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
  if (!aligned16(counts) || !aligned16(offsets) || !aligned16(perm_token) || !aligned16(inv) ||
      (perm_w && !aligned16(perm_w)))
    return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (moe::noalloc_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_permute(topk_idx, topk_w, x, T, d, E, k, dtype == MOE_BF16, counts,
                                        offsets, perm_token, inv, perm_w, x_perm, ws, stream));
}

size_t moe_ffn_workspace_size(int E, int rows, int d, int f) {
  return moe::ffn_workspace_bytes(E, rows, d, f);
}

size_t moe_workspace_size(int T, int d, int f, int E, int k, int dtype) {
  if (T < 0 || d <= 0 || f <= 0 || E < 1 || E > 256 || k < 1 || k > E || !dtype_ok(dtype))
    return 0;
  if ((long long)T * k >= (1ll << 31)) return 0;
  if (T == 0) return 0;  // every call is a no-op
  size_t need = moe::permute_workspace_bytes(T, E, k);
  need = std::max(need, moe::ffn_workspace_bytes(E, T * k, d, f));
  return need;
}

static int check_ffn_common(const int32_t* offsets, int E, int rows, int d, int f, int dtype,
                            void* workspace, size_t ws_bytes) {
  if (E < 1 || E > 256 || rows < 0 || d <= 0 || f <= 0) return MOE_ERR_INVALID;
  if ((long long)rows * (d > f ? d : f) >= (1ll << 40)) return MOE_ERR_INVALID;
  if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (!dims_ok(d) || !dims_ok(f)) return MOE_ERR_UNSUPPORTED;
  if (rows > 0 && !offsets) return MOE_ERR_INVALID;
  // the workspace is optional (it enables the GEMMs' tail split)
  if (workspace && !aligned16(workspace)) return MOE_ERR_UNSUPPORTED;
  (void)ws_bytes;
  return MOE_OK;
}

int moe_expert_up(const void* x, const int32_t* gather_idx, const int32_t* offsets, int E,
                  int rows, int d, int f, int dtype, const void* W_gate, const void* W_up,
                  void* a_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_ffn_common(offsets, E, rows, d, f, dtype, workspace, ws_bytes);
  if (st != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (!x || !W_gate || !W_up || !a_out) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(a_out) ||
      (gather_idx && !aligned16(gather_idx)) || !aligned16(offsets))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_expert_up(x, gather_idx, offsets, E, rows, d, f,
                                          dtype == MOE_BF16, W_gate, W_up, a_out, nullptr,
                                          nullptr, workspace, ws_bytes, stream));
}

int moe_expert_up_save(const void* x, const int32_t* gather_idx, const int32_t* offsets, int E,
                       int rows, int d, int f, int dtype, const void* W_gate, const void* W_up,
                       void* a_out, void* h_out, void* u_out, void* workspace, size_t ws_bytes,
                       hipStream_t stream) {
  int st = check_ffn_common(offsets, E, rows, d, f, dtype, workspace, ws_bytes);
  if (st != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (!x || !W_gate || !W_up || !a_out || !h_out || !u_out) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(a_out) ||
      !aligned16(h_out) || !aligned16(u_out) || (gather_idx && !aligned16(gather_idx)) ||
      !aligned16(offsets))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_expert_up(x, gather_idx, offsets, E, rows, d, f,
                                          dtype == MOE_BF16, W_gate, W_up, a_out, h_out, u_out,
                                          workspace, ws_bytes, stream));
}

int moe_expert_down(const void* a, const int32_t* offsets, int E, int rows, int f, int d,
                    int dtype, const void* W_down, float* y_perm, const int32_t* scatter_idx,
                    const float* row_w, float* y, void* workspace, size_t ws_bytes,
                    hipStream_t stream) {
  int st = check_ffn_common(offsets, E, rows, d, f, dtype, workspace, ws_bytes);
  if (st != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (!a || !W_down || (!y_perm && !y)) return MOE_ERR_INVALID;
  if (!aligned16(a) || !aligned16(W_down) || !aligned16(offsets) ||
      (y_perm && !aligned16(y_perm)) || (y && !aligned16(y)) ||
      (scatter_idx && !aligned16(scatter_idx)) || (row_w && !aligned16(row_w)))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_expert_down(a, offsets, E, rows, f, d, dtype == MOE_BF16, W_down,
                                            y_perm, scatter_idx, row_w, y, workspace, ws_bytes,
                                            stream));
}

int moe_ffn_forward(const void* x, const int32_t* gather_idx, const int32_t* offsets, int E,
                    int rows, int d, int f, int dtype, const void* W_gate, const void* W_up,
                    const void* W_down, void* a_buf, float* y_perm, const int32_t* scatter_idx,
                    const float* row_w, float* y, void* workspace, size_t ws_bytes,
                    hipStream_t stream) {
  int st = check_ffn_common(offsets, E, rows, d, f, dtype, workspace, ws_bytes);
  if (st != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  if (!x || !W_gate || !W_up || !W_down || !a_buf || (!y_perm && !y)) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down) ||
      !aligned16(a_buf) || !aligned16(offsets) || (gather_idx && !aligned16(gather_idx)) ||
      (y_perm && !aligned16(y_perm)) || (y && !aligned16(y)) ||
      (scatter_idx && !aligned16(scatter_idx)) || (row_w && !aligned16(row_w)))
    return MOE_ERR_UNSUPPORTED;
  const bool bf = dtype == MOE_BF16;
  hipError_t e = moe::launch_expert_up(x, gather_idx, offsets, E, rows, d, f, bf, W_gate, W_up,
                                       a_buf, nullptr, nullptr, workspace, ws_bytes, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_expert_down(a_buf, offsets, E, rows, f, d, bf, W_down, y_perm,
                                            scatter_idx, row_w, y, workspace, ws_bytes, stream));
}

int moe_combine(const float* y_perm, const int32_t* inv, const float* topk_w, int T, int d, int k,
                const float* y_shared, const float* shared_gate_logit, int accumulate, float* y,
                hipStream_t stream) {
  if (T < 0 || k < 1 || k > 256 || d <= 0) return MOE_ERR_INVALID;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_INVALID;
  if (accumulate != 0 && accumulate != 1) return MOE_ERR_INVALID;
  if (T == 0) return MOE_OK;
  if (!y) return MOE_ERR_INVALID;
  if (inv && (!y_perm || !topk_w)) return MOE_ERR_INVALID;
  if (shared_gate_logit && !y_shared) return MOE_ERR_INVALID;
  if (d % 8) return MOE_ERR_UNSUPPORTED;
  if ((inv && (!aligned16(y_perm) || !aligned16(inv) || !aligned16(topk_w))) || !aligned16(y) ||
      (y_shared && !aligned16(y_shared)))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_combine(y_perm, inv, topk_w, T, d, k, y_shared, shared_gate_logit,
                                        accumulate == 1, y, stream));
}

int moe_expert_down_f16(const void* a, const int32_t* offsets, int E, int rows, int f, int d,
                        const void* W_down, uint16_t* y_h, float* y_s, void* workspace,
                        size_t ws_bytes, hipStream_t stream) {
  int st = check_ffn_common(offsets, E, rows, d, f, MOE_BF16, workspace, ws_bytes);
  if (st != MOE_OK) return st;
  if (d % 32) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!a || !W_down || !y_h || !y_s) return MOE_ERR_INVALID;
  if (!aligned16(a) || !aligned16(W_down) || !aligned16(offsets) || !aligned16(y_h) ||
      !aligned16(y_s))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_expert_down_f16(a, offsets, E, rows, f, d, W_down, y_h, y_s,
                                                workspace, ws_bytes, stream));
}

int moe_combine_f16(const uint16_t* y_h, const float* y_s, const int32_t* inv, const float* topk_w,
                    int T, int d, int k, const uint16_t* ys_h, const float* ys_s,
                    const float* shared_gate_logit, int accumulate, float* y,
                    hipStream_t stream) {
  if (T < 0 || k < 1 || k > 256 || d <= 0) return MOE_ERR_INVALID;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_INVALID;
  if (accumulate != 0 && accumulate != 1) return MOE_ERR_INVALID;
  if (T == 0) return MOE_OK;
  if (!y) return MOE_ERR_INVALID;
  if (inv && (!y_h || !y_s || !topk_w)) return MOE_ERR_INVALID;
  if (!ys_h != !ys_s) return MOE_ERR_INVALID;
  if (shared_gate_logit && !ys_h) return MOE_ERR_INVALID;
  if (d % 32) return MOE_ERR_UNSUPPORTED;
  if ((inv && (!aligned16(y_h) || !aligned16(y_s) || !aligned16(inv) || !aligned16(topk_w))) ||
      !aligned16(y) || (ys_h && (!aligned16(ys_h) || !aligned16(ys_s))))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_combine_f16(y_h, y_s, inv, topk_w, T, d, k, ys_h, ys_s,
                                            shared_gate_logit, accumulate == 1, y, stream));
}

// ---------------------------------------------------------------- backward

int moe_combine_backward(const float* dy, const float* y_perm, const int32_t* inv,
                         const float* topk_w, int T, int d, int k, int dtype,
                         const float* y_shared, const float* shared_gate_logit, void* dy_perm,
                         float* dw, void* dy_shared, float* dgate_logit, hipStream_t stream) {
  if (T < 0 || k < 1 || k > 256 || d <= 0) return MOE_ERR_INVALID;
  if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_INVALID;
  if (T == 0) return MOE_OK;
  if (!dy || !y_perm || !inv || !topk_w || !dy_perm || !dw) return MOE_ERR_INVALID;
  if (shared_gate_logit && (!dy_shared || !y_shared || !dgate_logit)) return MOE_ERR_INVALID;
  if (dgate_logit && !shared_gate_logit) return MOE_ERR_INVALID;
  if (d % 8) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(dy) || !aligned16(y_perm) || !aligned16(inv) || !aligned16(topk_w) ||
      !aligned16(dy_perm) || !aligned16(dw) || (y_shared && !aligned16(y_shared)) ||
      (dy_shared && !aligned16(dy_shared)))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_combine_backward(dy, y_perm, inv, topk_w, T, d, k,
                                                 dtype == MOE_BF16, y_shared, shared_gate_logit,
                                                 dy_perm, dw, dy_shared, dgate_logit, stream));
}

int moe_combine_backward_f16(const float* dy, const uint16_t* y_h, const float* y_s,
                             const int32_t* inv, const float* topk_w, int T, int d, int k,
                             int dtype, const uint16_t* ys_h, const float* ys_s,
                             const float* shared_gate_logit, void* dy_perm, float* dw,
                             void* dy_shared, float* dgate_logit, hipStream_t stream) {
  if (T < 0 || k < 1 || k > 256 || d <= 0) return MOE_ERR_INVALID;
  if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_INVALID;
  if (T == 0) return MOE_OK;
  if (!dy || !y_h || !y_s || !inv || !topk_w || !dy_perm || !dw) return MOE_ERR_INVALID;
  if (!ys_h != !ys_s) return MOE_ERR_INVALID;
  if (shared_gate_logit && (!dy_shared || !ys_h || !dgate_logit)) return MOE_ERR_INVALID;
  if (dgate_logit && !shared_gate_logit) return MOE_ERR_INVALID;
  if (d % 32) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(dy) || !aligned16(y_h) || !aligned16(y_s) || !aligned16(inv) ||
      !aligned16(topk_w) || !aligned16(dy_perm) || !aligned16(dw) ||
      (ys_h && (!aligned16(ys_h) || !aligned16(ys_s))) || (dy_shared && !aligned16(dy_shared)))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_combine_backward_f16(
      dy, y_h, y_s, inv, topk_w, T, d, k, dtype == MOE_BF16, ys_h, ys_s, shared_gate_logit,
      dy_perm, dw, dy_shared, dgate_logit, stream));
}

static int check_bwd_common(const int32_t* offsets, int E, int rows, int d, int f, int dtype) {
  if (E < 1 || E > 256 || rows < 0 || d <= 0 || f <= 0) return MOE_ERR_INVALID;
  if ((long long)rows * 2 * (d > f ? d : f) >= (1ll << 40)) return MOE_ERR_INVALID;
  if ((long long)E * d * 2 * f >= (1ll << 40)) return MOE_ERR_INVALID;
  if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (!dims_ok(d) || !dims_ok(f)) return MOE_ERR_UNSUPPORTED;
  if (!offsets) return MOE_ERR_INVALID;
  if (!aligned16(offsets)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_ffn_backward_workspace_size(int E, int rows, int d, int f) {
  if (E < 1 || E > 256 || rows < 0 || d <= 0 || f <= 0) return 0;
  return moe::ffn_backward_workspace_bytes(E, rows, d, f);
}

int moe_expert_down_backward(const void* dy_perm, const int32_t* offsets, int E, int rows, int f,
                             int d, int dtype, const void* W_down, const void* h, const void* u,
                             const void* act, void* dhu, float* dW_down, void* workspace,
                             size_t ws_bytes, hipStream_t stream) {
  int st = check_bwd_common(offsets, E, rows, d, f, dtype);
  if (st != MOE_OK) return st;
  if (workspace && !aligned16(workspace)) return MOE_ERR_UNSUPPORTED;
  if (!workspace) ws_bytes = 0;
  if (!W_down || !dW_down) return MOE_ERR_INVALID;
  if (rows > 0 && (!dy_perm || !h || !u || !act || !dhu)) return MOE_ERR_INVALID;
  if (!aligned16(W_down) || !aligned16(dW_down) || (dy_perm && !aligned16(dy_perm)) ||
      (h && !aligned16(h)) || (u && !aligned16(u)) || (act && !aligned16(act)) ||
      (dhu && !aligned16(dhu)))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_expert_down_backward(dy_perm, offsets, E, rows, f, d,
                                                     dtype == MOE_BF16, W_down, h, u, act, dhu,
                                                     dW_down, workspace, ws_bytes, stream));
}

int moe_expert_up_backward(const void* x, const int32_t* gather_idx, const int32_t* offsets,
                           int E, int rows, int d, int f, int dtype, const void* W_gate,
                           const void* W_up, const void* dhu, float* dx_perm, int accumulate,
                           float* dW_gate, float* dW_up, void* workspace, size_t ws_bytes,
                           hipStream_t stream) {
  int st = check_bwd_common(offsets, E, rows, d, f, dtype);
  if (st != MOE_OK) return st;
  if (workspace && !aligned16(workspace)) return MOE_ERR_UNSUPPORTED;
  if (!workspace) ws_bytes = 0;
  if (accumulate != 0 && accumulate != 1) return MOE_ERR_INVALID;
  if (!W_gate || !W_up || !dW_gate || !dW_up) return MOE_ERR_INVALID;
  if (rows > 0 && (!x || !dhu || !dx_perm)) return MOE_ERR_INVALID;
  if (!aligned16(W_gate) || !aligned16(W_up) || !aligned16(dW_gate) || !aligned16(dW_up) ||
      (x && !aligned16(x)) || (dhu && !aligned16(dhu)) || (dx_perm && !aligned16(dx_perm)) ||
      (gather_idx && !aligned16(gather_idx)))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_expert_up_backward(x, gather_idx, offsets, E, rows, d, f,
                                                   dtype == MOE_BF16, W_gate, W_up, dhu, dx_perm,
                                                   accumulate, dW_gate, dW_up, workspace, ws_bytes,
                                                   stream));
}

int moe_unpermute(const float* dx_perm, const int32_t* inv, int T, int d, int k, int accumulate,
                  float* dx, hipStream_t stream) {
  if (T < 0 || k < 1 || k > 256 || d <= 0) return MOE_ERR_INVALID;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_INVALID;
  if (accumulate != 0 && accumulate != 1) return MOE_ERR_INVALID;
  if (T == 0) return MOE_OK;
  if (!dx_perm || !inv || !dx) return MOE_ERR_INVALID;
  if (d % 8) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(dx_perm) || !aligned16(inv) || !aligned16(dx)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_unpermute(dx_perm, inv, T, d, k, accumulate == 1, dx, stream));
}

int moe_topk_weights_backward(const float* logits, const int32_t* topk_idx, const float* dw, int T,
                              int E, int k, int score, float* dL, hipStream_t stream) {
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E) return MOE_ERR_INVALID;
  if ((long long)T * E >= (1ll << 31)) return MOE_ERR_INVALID;
  if (score != MOE_SOFTMAX_TOPK_RENORM && score != MOE_SOFTMAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !dw || !dL) return MOE_ERR_INVALID;
  return hip_status(moe::launch_topk_weights_backward(logits, topk_idx, dw, T, E, k,
                                                      score == MOE_SOFTMAX_TOPK_RENORM, dL,
                                                      stream));
}

size_t moe_linear_backward_workspace_size(int T, int d, int E) {
  if (T < 0 || d <= 0 || E < 1 || E > 256) return 0;
  return moe::linear_backward_workspace_bytes(T, d, E);
}

int moe_linear_backward(const void* x, const void* W, const float* G, int T, int d, int E,
                        int dtype, float* dW, float* db, float* dx, void* workspace,
                        size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || d <= 0 || E < 1 || E > 256) return MOE_ERR_INVALID;
  if ((long long)T * (d > E ? d : E) >= (1ll << 31)) return MOE_ERR_INVALID;
  if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!G || (dW && !x) || (dx && !W)) return MOE_ERR_INVALID;
  if (!dims_ok(d)) return MOE_ERR_UNSUPPORTED;
  if ((dW && !aligned16(x)) || (dx && !aligned16(dx))) return MOE_ERR_UNSUPPORTED;
  if (dW || dtype == MOE_BF16) {  // dW partials; bf16: G split into hi, lo
    const size_t need = moe::linear_backward_workspace_bytes(T, d, E);
    if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_UNSUPPORTED;
  }
  return hip_status(moe::launch_linear_backward(x, W, G, T, d, E, dtype == MOE_BF16, dW, db, dx,
                                                workspace, stream));
}

// ---------------------------------------------------------------- measurement

int moe_probe_mfma(int blocks, int iters, const void* operands, uint64_t* ticks,
                   hipStream_t stream) {
  if (blocks < 1 || blocks > (1 << 20) || iters < 1) return MOE_ERR_INVALID;
  if (!ticks) return MOE_ERR_INVALID;
  if (!aligned16(ticks) || (operands && !aligned16(operands))) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_probe_mfma(blocks, iters, operands, ticks, stream));
}

int moe_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes == 0) return MOE_OK;
  if (!src || !sink) return MOE_ERR_INVALID;
  if (bytes % 16 != 0 || !aligned16(src) || !aligned16(sink)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_probe_read(src, bytes, sink, stream));
}

}  // extern "C"
