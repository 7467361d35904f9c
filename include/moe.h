/*
 * moe.h -- C ABI of libmoe.so: the forward pass of a Mixture-of-Experts
 * expert layer on one MI355X (gfx950), on one GPU's share of tokens.
 *
 * The layer (what each call computes, and where the pages state it):
 *   - each token activates a sparse subset of E experts
 *       (DisagMoE technical summary, "1. Declaracao do Problema");
 *   - the subset is the router's top-k; tokens are dispatched to their
 *     experts and the expert outputs combined back
 *       (DisagMoE technical summary, "2.2 AF-Pipe", stage alignment);
 *   - experts are FFN layers ("2.1 Posicionamento de Componentes
 *     Desagregados") made of two GEMMs, "layer 0" over the token dimension
 *     M and "layer 1" over the hidden dimension N
 *       (COMET page, "COMET's Technical Principles", tensor decomposition).
 * The pages fix no score function or activation.  This library implements
 * a softmax router with optional renormalisation of the k selected weights,
 * and SwiGLU experts F_e(z) = (SiLU(z W_gate[e]) * (z W_up[e])) W_down[e],
 * SiLU(h) = h / (1 + exp(-h)), without biases.
 *
 * Conventions shared by every call:
 *   - every tensor pointer is a DEVICE pointer owned by the caller; tensors
 *     are dense and row-major; no call allocates, frees or keeps device
 *     memory between calls;
 *   - every call is asynchronous on the given stream (NULL = the null
 *     stream); arguments are validated on the host before anything is
 *     launched, and a rejected call launches nothing; a device fault
 *     surfaces at the caller's next synchronisation;
 *   - return value: MOE_OK, or an error code (see moe_status_string);
 *   - dtype MOE_BF16: x and weights bf16, accumulation fp32; MOE_F32: all
 *     fp32 (the small-layer path, plain FMA, not tuned for size);
 *   - limits: 1 <= k <= E <= 256; d, f > 0 and multiples of 8; T >= 0
 *     (T = 0 or rows = 0 is valid: nothing to compute, and moe_permute
 *     still writes zero counts and offsets); T*k < 2^31; pointers 16-byte
 *     aligned;
 *   - scratch memory comes from a caller-owned workspace whose size the
 *     matching *_workspace_size call returns.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* null required pointer, bad size, k > E, ... */
  MOE_ERR_UNSUPPORTED = 2, /* misaligned pointer, d or f not a multiple of 8, unknown enum */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than *_workspace_size */
  MOE_ERR_HIP = 4          /* a HIP launch failed */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };                          /* storage dtype */
enum { MOE_SOFTMAX_TOPK_RENORM = 0, MOE_SOFTMAX_TOPK = 1 };  /* router weights */

/* Human-readable text of a status code (static storage, never NULL). */
const char* moe_status_string(int status);

/*
 * moe_route -- router logits, top-k selection and weights.
 * Passage: top-k expert selection per token (DisagMoE technical summary,
 * "2.2 AF-Pipe"); sparse activation ("1. Declaracao do Problema").
 *   logits L[t,e] = sum_i x[t,i] W_r[i,e] + bias[e], fp32 accumulation;
 *   topk_idx[t, j]: the j-th expert of token t in the order (descending L,
 *     ascending expert index) -- exactly equal logits go to the lower index;
 *   topk_w[t, j] = p_sel / sum over the k picks of p (score RENORM) or p_sel
 *     (score TOPK), p = softmax over all E logits.
 * Arguments:
 *   x [T, d] (dtype), W_r [d, E] (dtype), bias [E] fp32 or NULL;
 *   topk_idx [T, k] int32 out; topk_w [T, k] fp32 out;
 *   logits_out [T, E] fp32 out or NULL: the exact logits the selection used.
 * The logits are summed in a fixed order: the call is deterministic.  It
 * needs no workspace: W_r is read in the layout given.  Every token gets k
 * distinct experts in [0, E) whatever its logits (a NaN logit ranks below
 * -inf and counts as -inf in the weights; a token whose logits are all NaN
 * gets NaN weights).
 */
int moe_route(const void* x, const void* W_r, const float* bias, int T, int d, int E, int k,
              int score, int dtype, int32_t* topk_idx, float* topk_w, float* logits_out,
              hipStream_t stream);

/* Workspace bytes moe_permute needs for T tokens, E experts, top-k. */
size_t moe_permute_workspace_size(int T, int E, int k);

/*
 * moe_permute -- dispatch: per-expert histogram, exclusive prefix scan and a
 * stable token permutation (the dispatch of DisagMoE technical summary,
 * "2.2 AF-Pipe"; the token fetch of COMET page, "COMET's Technical
 * Principles", computation rescheduling).
 *   counts[e]  = #{(t, j) : topk_idx[t, j] = e};
 *   offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e]  (offsets[E] = T*k);
 *   the pairs of expert e take rows offsets[e] .. offsets[e+1]-1 in
 *   ascending token order: perm_token[r] = t, inv[t, j] = r,
 *   perm_w[r] = topk_w[t, j];
 *   x_perm[r, :] = x[perm_token[r], :] when x_perm is not NULL (NULL: the
 *   gather is left to moe_expert_up, which reads x through perm_token).
 * Arguments: topk_idx [T, k] int32 with values in [0, E) (values outside are
 *   undefined behaviour) and the k experts of a token distinct, as
 *   moe_route produces them (an expert repeated in one token's list is
 *   counted once: both slots get the same row, offsets[E] < T*k, and every
 *   row below offsets[E] is still written, rows offsets[E] .. T*k-1 of
 *   perm_token, perm_w and x_perm are left untouched); topk_w [T, k] fp32
 *   or NULL (then perm_w must be NULL); x [T, d] (dtype) required only with
 *   x_perm; counts [E],
 *   offsets [E+1], perm_token [T*k], inv [T, k] int32 out; perm_w [T*k]
 *   fp32 out or NULL; x_perm [T*k, d] (dtype) out or NULL.
 * The result is deterministic (no atomics decide any order).
 */
int moe_permute(const int32_t* topk_idx, const float* topk_w, const void* x, int T, int d, int E,
                int k, int dtype, int32_t* counts, int32_t* offsets, int32_t* perm_token,
                int32_t* inv, float* perm_w, void* x_perm, void* workspace, size_t ws_bytes,
                hipStream_t stream);

/*
 * moe_permute_noalloc -- moe_permute without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation).  The same
 * arguments, results and status codes as moe_permute; its block tables live
 * in a static device array of 1 MiB per GPU instead (held until the process
 * ends), so it calls no allocator.  Limit: 2 * ceil(T / 256) * E int32 (each
 * table rounded up to 256 bytes) must fit 1 MiB -- e.g. T <= 131072 at
 * E = 256, T <= 1048576 at E = 32 -- else MOE_ERR_WORKSPACE and nothing is
 * launched.  Every byte the kernels read from the array is written earlier in
 * the same call.  Calls that overlap on one GPU (other streams, other host
 * threads) share the array and race: serialise them.
 */
int moe_permute_noalloc(const int32_t* topk_idx, const float* topk_w, const void* x, int T, int d,
                        int E, int k, int dtype, int32_t* counts, int32_t* offsets,
                        int32_t* perm_token, int32_t* inv, float* perm_w, void* x_perm,
                        hipStream_t stream);

/*
 * Workspace bytes that let moe_expert_up / moe_expert_down / moe_ffn_forward
 * split the K loop of the tiles of a mostly idle last round of tiles (the
 * partial sums of the split tiles are kept there and added in a fixed
 * order by a second pass, so results stay deterministic).  The workspace is
 * optional: with NULL or fewer bytes the GEMMs run unsplit.  One call's
 * workspace must not be used by another call running at the same time.
 */
size_t moe_ffn_workspace_size(int E, int rows, int d, int f);

/*
 * moe_workspace_size -- one workspace size that serves every forward call of
 * a layer with T tokens, model dim d, expert FFN dim f, E experts and top-k
 * (moe_permute, moe_expert_up / moe_expert_down / moe_ffn_forward with
 * rows = T*k; moe_route and moe_combine need none): the calls of one forward
 * run in order on one stream, so they can share one buffer of this many
 * bytes (16-byte aligned).  It is at least each of
 * moe_permute_workspace_size(T, E, k) and moe_ffn_workspace_size(E, T*k, d, f);
 * the FFN part does not depend on the shapes, so the same buffer also serves
 * a shared-expert FFN (E = 1, rows = T, any f).  Returns 0 for T = 0 (every
 * call is then a no-op that reads no workspace) and for arguments any call
 * would reject.  The buffer must not be shared by calls running at the same
 * time.
 */
size_t moe_workspace_size(int T, int d, int f, int E, int k, int dtype);

/*
 * moe_expert_up -- grouped GEMM "layer 0" with fused SwiGLU (COMET page,
 * "COMET's Technical Principles": the expert's first GEMM, over the token
 * dimension M; its tiles are walked M-first for each weight panel).
 * For every expert e and row r in [offsets[e], offsets[e+1]):
 *   z = x[gather_idx[r], :] (or x[r, :] when gather_idx is NULL),
 *   a_out[r, :] = SiLU(z W_gate[e]) * (z W_up[e]), stored in dtype (bf16
 *   rounds to nearest even).
 * Arguments: x [n_x, d]; gather_idx [rows] int32 or NULL, entries in
 *   [0, min(n_x, rows)) (others are undefined behaviour); offsets [E+1]
 *   int32 device (offsets[0] = 0, non-decreasing, offsets[E] = rows);
 *   W_gate, W_up [E, d, f]; a_out [rows, f] out.
 */
int moe_expert_up(const void* x, const int32_t* gather_idx, const int32_t* offsets, int E,
                  int rows, int d, int f, int dtype, const void* W_gate, const void* W_up,
                  void* a_out, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * moe_expert_up_save -- moe_expert_up that also keeps the two projections
 * for the backward pass (training: COMET page, "What Is COMET"):
 *   h_out[r, :] = z W_gate[e],  u_out[r, :] = z W_up[e]   (dtype, bf16 RNE),
 * with a_out as in moe_expert_up.  h_out, u_out [rows, f] out, both required.
 */
int moe_expert_up_save(const void* x, const int32_t* gather_idx, const int32_t* offsets, int E,
                       int rows, int d, int f, int dtype, const void* W_gate, const void* W_up,
                       void* a_out, void* h_out, void* u_out, void* workspace, size_t ws_bytes,
                       hipStream_t stream);

/*
 * moe_expert_down -- grouped GEMM "layer 1" (COMET page, "COMET's Technical
 * Principles": the expert's second GEMM, producing the hidden dimension N;
 * tiles are walked M-first for each weight panel) with an optional fused
 * top-k weighted combine
 * (DisagMoE technical summary, "2.2 AF-Pipe", combine).
 *   out[r, :] = a[r, :] W_down[e] for rows r of expert e;
 *   y_perm != NULL: y_perm[r, :] = out[r, :]  (fp32, deterministic);
 *   y != NULL:      y[scatter_idx[r], :] += row_w[r] * out[r, :]
 *                   (fp32 atomic adds: the summation order of the k
 *                   contributions of a token is not fixed; row_w NULL
 *                   means weight 1, scatter_idx NULL means row r -> r).
 * At least one of y_perm and y must be given.  y must be initialised by the
 * caller (zero, or a shared-expert output).
 * Arguments: a [rows, f] (dtype); offsets as in moe_expert_up;
 *   W_down [E, f, d]; y_perm [rows, d] fp32 or NULL; scatter_idx [rows]
 *   int32 or NULL; row_w [rows] fp32 or NULL; y [n_y, d] fp32 or NULL.
 */
int moe_expert_down(const void* a, const int32_t* offsets, int E, int rows, int f, int d,
                    int dtype, const void* W_down, float* y_perm, const int32_t* scatter_idx,
                    const float* row_w, float* y, void* workspace, size_t ws_bytes,
                    hipStream_t stream);

/*
 * moe_ffn_forward -- moe_expert_up followed by moe_expert_down on the same
 * stream (the expert FFN of DisagMoE technical summary, "2.1"; both GEMMs
 * of COMET page, "COMET's Technical Principles").  a_buf [rows, f] (dtype)
 * is the caller's buffer for the intermediate activation.
 */
int moe_ffn_forward(const void* x, const int32_t* gather_idx, const int32_t* offsets, int E,
                    int rows, int d, int f, int dtype, const void* W_gate, const void* W_up,
                    const void* W_down, void* a_buf, float* y_perm, const int32_t* scatter_idx,
                    const float* row_w, float* y, void* workspace, size_t ws_bytes,
                    hipStream_t stream);

/*
 * moe_combine -- top-k weighted combine / unpermute (DisagMoE technical
 * summary, "2.2 AF-Pipe", combine), plus an optional shared-expert term:
 *   v[t, :] = sum_j topk_w[t, j] * y_perm[inv[t, j], :]   (if inv != NULL)
 *             + g_t * y_shared[t, :]                      (if y_shared != NULL)
 *   g_t = 1 / (1 + exp(-shared_gate_logit[t])) (or 1 when the logit is NULL)
 *   y = v (accumulate = 0) or y += v (accumulate = 1).
 * With neither term, v = 0 (accumulate = 0 then clears y, e.g. before the
 * fused combine of moe_expert_down adds into it).
 * The k terms are summed in slot order: deterministic.
 * Arguments: y_perm [T*k, d] fp32, inv [T, k] int32 and topk_w [T, k] fp32,
 *   all three given or inv NULL; y_shared [T, d] fp32 or NULL;
 *   shared_gate_logit [T] fp32 or NULL; y [T, d] fp32 out.
 */
int moe_combine(const float* y_perm, const int32_t* inv, const float* topk_w, int T, int d, int k,
                const float* y_shared, const float* shared_gate_logit, int accumulate, float* y,
                hipStream_t stream);

/*
 * Compact layer-1 rows.  The same expert outputs as moe_expert_down's
 * y_perm, stored in half the bytes for the combine that reads them back:
 *   y_perm[r, c] = y_h[r, c] * y_s[r, c / 32],
 * y_h IEEE fp16 (round to nearest even), y_s one power of two per 32-column
 * row segment, chosen so that the segment's largest finite magnitude lands
 * in [2^14, 2^15): no value overflows fp16 and each keeps 11 significant
 * bits at its segment's scale (error at most 2^-11 of the segment's largest
 * magnitude; inf and NaN are kept).  The pages fix no storage precision for
 * this intermediate (DisagMoE technical summary, "2.2 AF-Pipe": the expert
 * outputs go back to be combined); the fp32 calls above stay the exact form.
 *
 * moe_expert_down_f16 -- moe_expert_down with this output (no fused combine):
 *   out[r, :] = a[r, :] W_down[e] for rows r of expert e, stored as above.
 * Arguments: a [rows, f] bf16; offsets, E, rows, f, workspace as in
 *   moe_expert_down; W_down [E, f, d] bf16; y_h [rows, d] (fp16 bits) out;
 *   y_s [rows, d / 32] fp32 out.  bf16 only and d a multiple of 32, else
 *   MOE_ERR_UNSUPPORTED.
 */
int moe_expert_down_f16(const void* a, const int32_t* offsets, int E, int rows, int f, int d,
                        const void* W_down, uint16_t* y_h, float* y_s, void* workspace,
                        size_t ws_bytes, hipStream_t stream);

/*
 * moe_combine_f16 -- moe_combine over compact rows: the same v and y, with
 *   y_perm[r, :] read as y_h[r, :] * y_s[r, : / 32] and y_shared[t, :] as
 *   ys_h[t, :] * ys_s[t, : / 32] (e.g. the shared experts' moe_expert_down_f16
 *   over T rows).  Each term is the product moe_combine forms from the
 *   restored value, in the same slot order: given the same rows, both calls
 *   write the same bits.
 * Arguments: y_h [T*k, d] fp16 bits and y_s [T*k, d / 32] fp32, inv [T, k]
 *   and topk_w [T, k] as in moe_combine (all four given or inv NULL);
 *   ys_h [T, d] and ys_s [T, d / 32], both or neither; shared_gate_logit [T]
 *   or NULL (needs ys_h); accumulate 0 or 1; y [T, d] fp32 out.  d a multiple
 *   of 32, else MOE_ERR_UNSUPPORTED.
 */
int moe_combine_f16(const uint16_t* y_h, const float* y_s, const int32_t* inv, const float* topk_w,
                    int T, int d, int k, const uint16_t* ys_h, const float* ys_s,
                    const float* shared_gate_logit, int accumulate, float* y, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward pass (training).  The pages train MoE models (COMET page, "What
 * Is COMET"; DisagMoE technical summary, "2.2 AF-Pipe", whose pipeline has
 * a backward stream); the calls below give the exact gradients of the
 * forward calls above for an upstream gradient dy of y, in reverse order:
 *   moe_combine_backward -> moe_expert_down_backward -> moe_expert_up_backward
 *   -> moe_unpermute; moe_topk_weights_backward -> moe_linear_backward
 *   (router: G = dL, W = W_r; gated shared expert: G = dgate, W = w_s).
 * Conventions as above (device pointers owned by the caller, asynchronous,
 * host validation first, no allocation); bf16 or fp32 storage as in the
 * forward (fp32: plain FMA kernels for small layers, as the forward's fp32
 * path); every sum in a fixed order (deterministic).
 * ------------------------------------------------------------------------ */

/*
 * moe_combine_backward -- gradient of moe_combine (DisagMoE technical
 * summary, "2.2 AF-Pipe", combine):
 *   dw[t, j] = <dy[t, :], y_perm[inv[t, j], :]>,
 *   dy_perm[inv[t, j], :] = topk_w[t, j] * dy[t, :]              (dtype; bf16 RNE);
 *   shared term (dy_shared != NULL): dy_shared[t, :] = g_t * dy[t, :] (dtype),
 *     g_t = sigmoid(shared_gate_logit[t]) or 1 when the logit is NULL;
 *     with the logit and y_shared: dgate_logit[t] = <dy[t], y_shared[t]> g_t (1 - g_t).
 * Arguments: dy [T, d] fp32; y_perm [T*k, d] fp32 (the forward's);
 *   inv, topk_w [T, k]; y_shared [T, d] fp32 (ungated shared output of the
 *   forward) or NULL; shared_gate_logit [T] or NULL; dy_perm [T*k, d] out in
 *   dtype (the storage dtype of the layer); dw [T, k] fp32 out; dy_shared
 *   [T, d] out in dtype or NULL; dgate_logit [T] fp32 out (required with the
 *   logit) or NULL.  1 <= k <= 256 (above 8 the slots are taken one after
 *   another, with the same summation order).
 */
int moe_combine_backward(const float* dy, const float* y_perm, const int32_t* inv,
                         const float* topk_w, int T, int d, int k, int dtype,
                         const float* y_shared,
                         const float* shared_gate_logit, void* dy_perm, float* dw,
                         void* dy_shared, float* dgate_logit, hipStream_t stream);

/*
 * moe_combine_backward_f16 -- moe_combine_backward over compact rows (the
 *   output of moe_expert_down_f16): the same gradients, with y_perm[r, :]
 *   read as y_h[r, :] * y_s[r, : / 32] and y_shared[t, :] as
 *   ys_h[t, :] * ys_s[t, : / 32].  dy_perm and dy_shared are the same values
 *   as moe_combine_backward's; dw and dgate_logit may differ from them in
 *   rounding order only (8 columns per step instead of 4).
 * Arguments: dy [T, d] fp32; y_h [T*k, d] fp16 bits, y_s [T*k, d / 32] fp32;
 *   inv, topk_w [T, k]; ys_h [T, d] and ys_s [T, d / 32], both or neither
 *   (the ungated shared output; needed with the logit); shared_gate_logit,
 *   dy_perm, dw, dy_shared, dgate_logit as in moe_combine_backward.
 *   1 <= k <= 256; d a multiple of 32, else MOE_ERR_UNSUPPORTED.
 */
int moe_combine_backward_f16(const float* dy, const uint16_t* y_h, const float* y_s,
                             const int32_t* inv, const float* topk_w, int T, int d, int k,
                             int dtype, const uint16_t* ys_h, const float* ys_s,
                             const float* shared_gate_logit, void* dy_perm, float* dw,
                             void* dy_shared, float* dgate_logit, hipStream_t stream);

/*
 * moe_expert_down_backward -- gradients of moe_expert_down (layer 1) and of
 * the SwiGLU of moe_expert_up, per expert e and row r of e:
 *   dA = dy_perm[r] W_down[e]^T,  s = sigmoid(h[r]),
 *   dhu[r, 0:f]  = dA * u[r] * s (1 + h[r] (1 - s))     (dH, dtype),
 *   dhu[r, f:2f] = dA * h[r] * s                        (dU, dtype),
 *   dW_down[e]   = sum_{r of e} act[r]^T dy_perm[r]     (fp32; 0 for empty experts).
 * Arguments: dy_perm [rows, d] (dtype); offsets as in moe_expert_up; W_down
 *   [E, f, d]; h, u [rows, f] (moe_expert_up_save); act [rows, f] (its
 *   a_out); dhu [rows, 2f] out (dtype); dW_down [E, f, d] fp32 out;
 *   workspace of moe_ffn_backward_workspace_size(E, rows, d, f) bytes or
 *   NULL (optional: with it, a launch with fewer weight-gradient tiles than
 *   about two per compute unit, such as the shared experts run as one
 *   expert, cuts each expert's rows into chunks whose fp32 partials are
 *   added in chunk order; the results stay deterministic either way).
 */
int moe_expert_down_backward(const void* dy_perm, const int32_t* offsets, int E, int rows, int f,
                             int d, int dtype, const void* W_down, const void* h, const void* u,
                             const void* act, void* dhu, float* dW_down, void* workspace,
                             size_t ws_bytes, hipStream_t stream);

/* Bytes of the optional workspace of moe_expert_down_backward and
 * moe_expert_up_backward (0 when no split would be used). */
size_t moe_ffn_backward_workspace_size(int E, int rows, int d, int f);

/*
 * moe_expert_up_backward -- gradients of moe_expert_up (layer 0) given dhu:
 *   dx_perm[r] (+)= dhu[r, 0:f] W_gate[e]^T + dhu[r, f:2f] W_up[e]^T   (fp32),
 *   dW_gate[e] = sum_{r of e} z_r^T dhu[r, 0:f],  dW_up[e] = sum z_r^T dhu[r, f:2f]
 *   (fp32; 0 for empty experts), z_r = x[gather_idx[r]] (or x[r]).
 * Arguments: x, gather_idx, offsets, W_gate, W_up as in moe_expert_up; dhu
 *   [rows, 2f] (dtype); dx_perm [rows, d] fp32 out (added to when
 *   accumulate = 1); dW_gate, dW_up [E, d, f] fp32 out; workspace as in
 *   moe_expert_down_backward (not used with a row gather).
 */
int moe_expert_up_backward(const void* x, const int32_t* gather_idx, const int32_t* offsets,
                           int E, int rows, int d, int f, int dtype, const void* W_gate,
                           const void* W_up, const void* dhu, float* dx_perm, int accumulate,
                           float* dW_gate, float* dW_up, void* workspace, size_t ws_bytes,
                           hipStream_t stream);

/*
 * moe_unpermute -- gradient of the dispatch (DisagMoE technical summary,
 * "2.2 AF-Pipe", dispatch): dx[t, :] (+)= sum_j dx_perm[inv[t, j], :] in slot
 * order.  dx_perm [T*k, d] fp32, inv [T, k], dx [T, d] fp32 out (added to
 * when accumulate = 1); 1 <= k <= 256.
 */
int moe_unpermute(const float* dx_perm, const int32_t* inv, int T, int d, int k, int accumulate,
                  float* dx, hipStream_t stream);

/*
 * moe_topk_weights_backward -- gradient of the top-k weights of moe_route
 * with respect to the logits, at the forward's selection (the selection
 * itself is piecewise constant):
 *   score RENORM: dL[t, e_j] = w_j (dw_j - sum_i w_i dw_i), 0 elsewhere;
 *   score TOPK:   dL[t, e] = p_e ([e = e_j] dw_j - sum_i p_{e_i} dw_i).
 * The weights are recomputed in fp32 from logits (moe_route's logits_out).
 * Arguments: logits [T, E] fp32, topk_idx [T, k], dw [T, k] fp32, dL [T, E] fp32 out.
 */
int moe_topk_weights_backward(const float* logits, const int32_t* topk_idx, const float* dw, int T,
                              int E, int k, int score, float* dL, hipStream_t stream);

/*
 * moe_linear_backward -- gradients of the skinny map L = x W (+ b) of the
 * router (DisagMoE technical summary, "2.2 AF-Pipe": top-k router) or of
 * the shared expert's gate, given G = dL [T, E]:
 *   dW = x^T G (fp32, summed over token chunks in order),
 *   db = sum_t G[t]   (if db != NULL),
 *   dx += G W^T       (if dx != NULL; fp32, added to).
 * Arguments: x [T, d] (dtype), W [d, E] (dtype), G [T, E] fp32, dW [d, E]
 *   fp32 out or NULL, db [E] fp32 out or NULL, dx [T, d] fp32 in/out or NULL;
 *   workspace of moe_linear_backward_workspace_size(T, d, E) bytes, 16-byte
 *   aligned (when dW, and always for bf16; MOE_ERR_WORKSPACE if missing or
 *   smaller).
 * bf16: both products run on the matrix cores with G entering as hi + lo,
 *   hi = bf16(G), lo = bf16(G - hi) (|G - hi - lo| <= 2^-18 |G|; each
 *   product is exact in the fp32 accumulators); fp32: plain fp32 FMA.
 * Requirements: 1 <= E <= 256; d a multiple of 8 and x, dx 16-byte aligned
 * (MOE_ERR_UNSUPPORTED otherwise: x rows and dx rows move as 16-byte vectors).
 * Every sum runs in a fixed order: the results are deterministic.
 */
size_t moe_linear_backward_workspace_size(int T, int d, int E);
int moe_linear_backward(const void* x, const void* W, const float* G, int T, int d, int E,
                        int dtype, float* dW, float* db, float* dx, void* workspace,
                        size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Measurement.  Kernel rates are reported as fractions of the chip's peaks
 * (the pages compare layer times across token lengths and expert loads:
 * COMET page, "COMET's Performance"); these calls measure the bf16 matrix
 * peak the chip sustains, and its shader clock, under an all-compute-unit
 * load, and the rate of a pure streaming read of a given size, to set
 * beside the datasheet figures.
 * ------------------------------------------------------------------------ */

/*
 * moe_probe_mfma -- `blocks` workgroups of 4 wave64s each run `iters` rounds
 * of 32 bf16 MFMAs of 16 x 16 x 32 (16384 flops each) on register operands
 * into 16 accumulators, so the launch performs blocks * 4 * iters * 32 *
 * 16384 flops (time it with events on the stream).  operands: NULL, or
 * device bf16 values, blocks * 16 * 256 vectors of 8 (blocks * 65536 bytes,
 * 16-byte aligned): every thread loads 8 A and 8 B vectors once and the
 * MFMAs cycle through them, so consecutive MFMAs multiply different bits (the
 * switching of a real GEMM's operands; NULL: fixed per-lane values).  The
 * values never reach memory and only need to be finite.  ticks [3 * blocks]
 * uint64 device out: per block, the shader-clock ticks and the 100 MHz
 * real-time ticks its wave 0 spent in the loop, and a word that is always 0.
 * MOE_ERR_INVALID for blocks outside [1, 2^20], iters < 1 or a NULL ticks;
 * MOE_ERR_UNSUPPORTED for a misaligned ticks or operands.
 */
int moe_probe_mfma(int blocks, int iters, const void* operands, uint64_t* ticks,
                   hipStream_t stream);

/*
 * moe_probe_read -- reads `bytes` bytes of device memory at src once, in
 * 16-byte non-temporal loads at a grid stride (at most 2048 workgroups of
 * 256 threads, four loads in flight per thread), and writes nothing but, in practice
 * never, one word at sink.  Time it with events on the stream: bytes / time
 * is the rate a pure streaming read reaches at that size, the reference for
 * a memory-bound stage of the same byte count.  src and sink device, 16-byte
 * aligned; bytes a multiple of 16 (MOE_ERR_UNSUPPORTED otherwise); bytes = 0
 * is a no-op; MOE_ERR_INVALID for a NULL src or sink.
 */
int moe_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
