"""Drive one MoE expert-layer forward through the C ABI.

Allocates the buffers of the path once (torch is used for device memory and
the stream only) and issues the C-ABI calls in order:

    moe_route -> moe_permute -> [shared experts] -> moe_expert_up
              -> moe_expert_down -> [moe_combine]

Two independent choices shape the path:

* gather: "fused" -- the layer-0 GEMM reads token rows of x through the
  permutation (no permuted copy of x); "copy" -- moe_permute writes x_perm.
* combine: "separate" -- the layer-1 GEMM writes y_perm (fp32) and
  moe_combine sums each token's k rows in slot order (deterministic);
  "separate16" -- the same with y_perm in its compact form (fp16 and one
  power-of-two factor per 32-column row segment: moe_expert_down_f16,
  moe_combine_f16; half the bytes of the round trip, the shared experts'
  output likewise); "atomic" -- the layer-1 epilogue adds w * out straight
  into y with fp32 atomic adds (no y_perm; the order of a token's k adds is
  not fixed).

Paths: "fast" = fused gather + separate16 combine (the benchmarked default,
deterministic; bf16 layers with d a multiple of 32, the fp32 y_perm
otherwise); "fast32" = fused gather + separate combine;
"atomic" = fused gather + atomic combine; "reference" = copy gather +
separate combine.

Training (``train=True``): the forward also keeps the layer-0 projections
h = x W_gate and u = x W_up (routed and shared) and the router logits, and
``backward(dy)`` issues the backward C-ABI calls in reverse order:

    moe_combine_backward[_f16] -> moe_expert_down_backward -> moe_expert_up_backward
    -> moe_unpermute -> moe_topk_weights_backward -> moe_linear_backward
    [-> shared experts: moe_expert_down_backward, moe_expert_up_backward,
        moe_linear_backward for the gate]

leaving the gradients in ``self.grads`` (fp32 device tensors).  Training
needs a deterministic separate combine (the combine backward reads the
forward's rows: y_perm, or its compact form on the "fast" path), keeps the backward's
intermediates in the layer's storage dtype (bf16 or fp32), and
always has moe_permute write x_perm: the layer-0 weight gradient reads the
expert's token rows in order from it (the forward GEMMs still read x
through the permutation on the "fast" path: x, T rows, stays in the
last-level cache where x_perm, T k rows, may not).

Shared experts: the n_s experts are stored side by side (gate/up projections
[d, n_s*f_s], down projections [n_s*f_s, d]), so their sum is one SwiGLU FFN
of width n_s*f_s, run as a single-expert FFN over x (offsets {0, T}).  With
the separate combine its output goes to a [T, d] buffer that moe_combine adds
(scaled per token by sigmoid(x . w_s) in the gated variant, its gate logit
from moe_route with E = 1); with the atomic combine it initialises y.
"""
from __future__ import annotations

import torch

from . import _lib as L
from .inputs import LayerConfig

PATHS = {"fast": ("fused", "separate16"), "fast32": ("fused", "separate"),
         "atomic": ("fused", "atomic"), "reference": ("copy", "separate")}


class MoeLayer:
    def __init__(self, cfg: LayerConfig, layer: dict, fused=None, keep_logits: bool = True,
                 path: str = "fast", train: bool = False):
        if fused is not None:  # shorthand kept for callers of the two original paths
            path = "atomic" if fused else "reference"
        self.path = path
        self.gather, self.comb = PATHS[path]
        self.train = train
        # the compact rows: bf16 layers whose d splits into 32-column segments
        if self.comb == "separate16" and (cfg.dtype != "bf16" or cfg.d % 32):
            self.comb = "separate"
        if train:
            if self.comb not in ("separate", "separate16"):
                raise ValueError("training needs the separate combine")
            keep_logits = True
        self.cfg = cfg
        self.t = layer
        dev = layer["x"].device
        T, d, f, E, k = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k
        R = T * k
        self.dtype = L.MOE_BF16 if cfg.dtype == "bf16" else L.MOE_F32
        act = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        i32, f32 = torch.int32, torch.float32
        e = lambda *s, dt=f32: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        self.idx = e(T, k, dt=i32)
        self.w = e(T, k)
        self.logits = e(T, E) if keep_logits else None
        self.counts = e(E, dt=i32)
        self.offsets = e(E + 1, dt=i32)
        self.perm_token = e(R, dt=i32)
        self.inv = e(T, k, dt=i32)
        self.perm_w = e(R)
        self.x_perm = e(R, d, dt=act) if (self.gather == "copy" or train) else None
        self.a = e(R, f, dt=act)
        self.y_perm = e(R, d) if self.comb == "separate" else None
        if self.comb == "separate16":
            self.y_h = e(R, d, dt=torch.float16)
            self.y_s = e(R, d // 32)
        self.y = e(T, d)
        self.ws_perm_bytes = L.moe_permute_workspace_size(T, E, k)
        self.ws_perm = e(max(self.ws_perm_bytes, 16), dt=torch.uint8)
        self.ws_ffn_bytes = L.moe_ffn_workspace_size(E, R, d, f)
        self.ws_ffn = e(max(self.ws_ffn_bytes, 16), dt=torch.uint8)
        if train:
            self.h = e(R, f, dt=act)
            self.u = e(R, f, dt=act)
        # shared experts
        self.ns = cfg.n_shared
        if self.ns:
            self.fs_all = self.ns * cfg.f_shared   # width of the side-by-side FFN
            self.s_a = e(T, self.fs_all, dt=act)
            self.s_offsets = torch.tensor([0, T], dtype=i32, device=dev)
            self.s_ws_bytes = L.moe_ffn_workspace_size(1, T, d, self.fs_all)
            self.s_ws = e(max(self.s_ws_bytes, 16), dt=torch.uint8)
            if train:
                self.s_h = e(T, self.fs_all, dt=act)
                self.s_u = e(T, self.fs_all, dt=act)
            if self.comb == "separate16":   # shared-expert output, compact
                self.ys_h = e(T, d, dt=torch.float16)
                self.ys_s = e(T, d // 32)
            elif not (self.comb == "atomic" and not cfg.shared_gated):
                self.ys = e(T, d)   # shared-expert output
            if cfg.shared_gated:
                self.g_idx = e(T, 1, dt=i32)
                self.g_w = e(T, 1)
                self.g_logit = e(T, 1)
                self.w_s_col = layer["w_s"].reshape(d, 1).contiguous()

    # -- stages ------------------------------------------------------------
    def route(self, stream=None):
        c, t = self.cfg, self.t
        score = L.MOE_SOFTMAX_TOPK_RENORM if c.renorm else L.MOE_SOFTMAX_TOPK
        L.moe_route(t["x"], t["W_r"], t.get("b"), c.T, c.d, c.E, c.k, score, self.dtype,
                    self.idx, self.w, self.logits, stream=stream)

    def permute(self, stream=None):
        c, t = self.cfg, self.t
        L.moe_permute(self.idx, self.w, t["x"], c.T, c.d, c.E, c.k, self.dtype, self.counts,
                      self.offsets, self.perm_token, self.inv, self.perm_w, self.x_perm,
                      self.ws_perm, self.ws_perm_bytes, stream=stream)

    def shared(self, stream=None):
        """Shared-expert output (and, with the atomic combine, y initialised
        with it, or cleared when there are none)."""
        c, t = self.cfg, self.t
        T, d = c.T, c.d
        if not self.ns:
            if self.comb == "atomic":
                L.moe_combine(None, None, None, T, d, c.k, None, None, 0, self.y, stream=stream)
            return
        fs = self.fs_all
        if c.shared_gated:
            # gate logit x . w_s (a one-column router)
            L.moe_route(t["x"], self.w_s_col, None, T, d, 1, 1, L.MOE_SOFTMAX_TOPK, self.dtype,
                        self.g_idx, self.g_w, self.g_logit, stream=stream)
        if self.train:
            L.moe_expert_up_save(t["x"], None, self.s_offsets, 1, T, d, fs, self.dtype,
                                 t["Ws_gate"], t["Ws_up"], self.s_a, self.s_h, self.s_u, self.s_ws,
                                 self.s_ws_bytes, stream=stream)
        else:
            L.moe_expert_up(t["x"], None, self.s_offsets, 1, T, d, fs, self.dtype, t["Ws_gate"],
                            t["Ws_up"], self.s_a, self.s_ws, self.s_ws_bytes, stream=stream)
        if self.comb == "separate16":
            L.moe_expert_down_f16(self.s_a, self.s_offsets, 1, T, fs, d, t["Ws_down"], self.ys_h,
                                  self.ys_s, self.s_ws, self.s_ws_bytes, stream=stream)
            return
        # ungated with the atomic combine: the output initialises y directly
        out = self.y if (self.comb == "atomic" and not c.shared_gated) else self.ys
        L.moe_expert_down(self.s_a, self.s_offsets, 1, T, fs, d, self.dtype, t["Ws_down"],
                          out, None, None, None, self.s_ws, self.s_ws_bytes, stream=stream)
        if self.comb == "atomic" and c.shared_gated:  # y = g * S(x); the routed part adds in later
            L.moe_combine(None, None, None, T, d, c.k, self.ys, self.g_logit, 0, self.y,
                          stream=stream)

    def expert_up(self, stream=None):
        c, t = self.cfg, self.t
        R = c.T * c.k
        if self.gather == "fused":
            src, gidx = t["x"], self.perm_token
        else:
            src, gidx = self.x_perm, None
        if self.train:
            L.moe_expert_up_save(src, gidx, self.offsets, c.E, R, c.d, c.f, self.dtype,
                                 t["W_gate"], t["W_up"], self.a, self.h, self.u, self.ws_ffn,
                                 self.ws_ffn_bytes, stream=stream)
        else:
            L.moe_expert_up(src, gidx, self.offsets, c.E, R, c.d, c.f, self.dtype, t["W_gate"],
                            t["W_up"], self.a, self.ws_ffn, self.ws_ffn_bytes, stream=stream)

    def expert_down(self, stream=None):
        c, t = self.cfg, self.t
        R = c.T * c.k
        if self.comb == "atomic":
            L.moe_expert_down(self.a, self.offsets, c.E, R, c.f, c.d, self.dtype, t["W_down"],
                              None, self.perm_token, self.perm_w, self.y, self.ws_ffn,
                              self.ws_ffn_bytes, stream=stream)
        elif self.comb == "separate16":
            L.moe_expert_down_f16(self.a, self.offsets, c.E, R, c.f, c.d, t["W_down"], self.y_h,
                                  self.y_s, self.ws_ffn, self.ws_ffn_bytes, stream=stream)
        else:
            L.moe_expert_down(self.a, self.offsets, c.E, R, c.f, c.d, self.dtype, t["W_down"],
                              self.y_perm, None, None, None, self.ws_ffn, self.ws_ffn_bytes,
                              stream=stream)

    def combine(self, stream=None):
        if self.comb == "atomic":
            return
        c = self.cfg
        T = c.T
        gl = self.g_logit if (self.ns and c.shared_gated) else None
        if self.comb == "separate16":
            ys_h, ys_s = (self.ys_h, self.ys_s) if self.ns else (None, None)
            L.moe_combine_f16(self.y_h, self.y_s, self.inv, self.w, T, c.d, c.k, ys_h, ys_s, gl,
                              0, self.y, stream=stream)
            return
        ys = self.ys if self.ns else None
        L.moe_combine(self.y_perm, self.inv, self.w, T, c.d, c.k, ys, gl, 0, self.y,
                      stream=stream)

    STAGES = ("route", "permute", "shared", "expert_up", "expert_down", "combine")

    def forward(self, stream=None, marks=None):
        """Run every stage; ``marks(name)`` (if given) is called after each
        stage, e.g. to record an event on the stream."""
        for name in self.STAGES:
            getattr(self, name)(stream)
            if marks is not None:
                marks(name)
        return self.y

    def capture_graph(self):
        """Record one forward pass into a HIP graph (a torch.cuda.CUDAGraph)
        over this layer's buffers and inputs, after one eager pass on a side
        stream (default priority); ``graph.replay()`` then reruns the whole
        path on whatever the input buffers hold, writing the same buffers.
        Every C-ABI call of the path is asynchronous on the calling stream,
        allocates nothing and synchronises nothing, which is what lets the
        capture record it; no call records a memset."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.forward()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self.forward()
        torch.cuda.synchronize()
        return g

    # -- backward ----------------------------------------------------------
    BSTAGES = ("combine_bwd", "expert_down_bwd", "expert_up_bwd", "unpermute", "router_bwd",
               "shared_bwd")

    def _alloc_backward(self):
        if getattr(self, "_bwd_ready", False):
            return
        c, t = self.cfg, self.t
        dev = t["x"].device
        T, d, f, E, k = c.T, c.d, c.f, c.E, c.k
        R = T * k
        f32 = torch.float32
        act = torch.bfloat16 if c.dtype == "bf16" else f32
        e = lambda *sh, dt=f32: torch.empty(*sh, dtype=dt, device=dev)  # noqa: E731
        self.dy_perm = e(R, d, dt=act)
        self.dw = e(T, k)
        self.dhu = e(R, 2 * f, dt=act)
        self.dx_perm = e(R, d)
        self.dL = e(T, E)
        g = dict(dx=e(T, d), dW_r=e(d, E), dW_gate=e(E, d, f), dW_up=e(E, d, f),
                 dW_down=e(E, f, d), db=e(E) if t.get("b") is not None else None)
        # the backward GEMMs' optional workspace (K-split partials of weight
        # gradients with few tiles: here the shared experts, one expert over T rows)
        need = L.moe_ffn_backward_workspace_size(E, R, d, f)
        if self.ns:
            need = max(need, L.moe_ffn_backward_workspace_size(1, T, d, self.fs_all))
        self.ws_bwd_bytes = need
        self.ws_bwd = e(max(need, 16), dt=torch.uint8)
        self.ws_lin_bytes = L.moe_linear_backward_workspace_size(T, d, E)
        self.ws_lin = e(max(self.ws_lin_bytes, 16), dt=torch.uint8)
        if self.ns:
            fs = self.fs_all
            self.dys = e(T, d, dt=act)
            self.s_dhu = e(T, 2 * fs, dt=act)
            g.update(dWs_gate=e(d, fs), dWs_up=e(d, fs), dWs_down=e(fs, d))
            if c.shared_gated:
                self.dgl = e(T, 1)
                g["dw_s"] = e(d, 1)
                self.ws_lin1_bytes = L.moe_linear_backward_workspace_size(T, d, 1)
                self.ws_lin1 = e(max(self.ws_lin1_bytes, 16), dt=torch.uint8)
        self.grads = g
        self._bwd_ready = True

    def backward(self, dy, stream=None, marks=None):
        """Gradients of <dy, y> for the last forward (``train=True``); ``marks``
        as in ``forward``, after each backward stage."""
        if not self.train:
            raise RuntimeError("construct the layer with train=True to run the backward")
        self._alloc_backward()
        c, t, g = self.cfg, self.t, self.grads
        T, d, f, E, k = c.T, c.d, c.f, c.E, c.k
        R = T * k
        mk = (lambda n: marks(n)) if marks is not None else (lambda n: None)
        gated = bool(self.ns and c.shared_gated)
        if self.comb == "separate16":
            ys_h, ys_s = (self.ys_h, self.ys_s) if gated else (None, None)
            L.moe_combine_backward_f16(dy, self.y_h, self.y_s, self.inv, self.w, T, d, k,
                                       self.dtype, ys_h, ys_s, self.g_logit if gated else None,
                                       self.dy_perm, self.dw, self.dys if self.ns else None,
                                       self.dgl if gated else None, stream=stream)
        else:
            L.moe_combine_backward(dy, self.y_perm, self.inv, self.w, T, d, k, self.dtype,
                                   self.ys if gated else None, self.g_logit if gated else None,
                                   self.dy_perm, self.dw, self.dys if self.ns else None,
                                   self.dgl if gated else None, stream=stream)
        mk("combine_bwd")
        L.moe_expert_down_backward(self.dy_perm, self.offsets, E, R, f, d, self.dtype,
                                   t["W_down"], self.h, self.u, self.a, self.dhu, g["dW_down"],
                                   self.ws_bwd, self.ws_bwd_bytes, stream=stream)
        mk("expert_down_bwd")
        L.moe_expert_up_backward(self.x_perm, None, self.offsets, E, R, d, f, self.dtype,
                                 t["W_gate"], t["W_up"], self.dhu, self.dx_perm, 0, g["dW_gate"],
                                 g["dW_up"], self.ws_bwd, self.ws_bwd_bytes, stream=stream)
        mk("expert_up_bwd")
        L.moe_unpermute(self.dx_perm, self.inv, T, d, k, 0, g["dx"], stream=stream)
        mk("unpermute")
        score = L.MOE_SOFTMAX_TOPK_RENORM if c.renorm else L.MOE_SOFTMAX_TOPK
        L.moe_topk_weights_backward(self.logits, self.idx, self.dw, T, E, k, score, self.dL,
                                    stream=stream)
        L.moe_linear_backward(t["x"], t["W_r"], self.dL, T, d, E, self.dtype, g["dW_r"],
                              g["db"], g["dx"], self.ws_lin, self.ws_lin_bytes, stream=stream)
        mk("router_bwd")
        if self.ns:
            fs = self.fs_all
            L.moe_expert_down_backward(self.dys, self.s_offsets, 1, T, fs, d, self.dtype,
                                       t["Ws_down"], self.s_h, self.s_u, self.s_a, self.s_dhu,
                                       g["dWs_down"], self.ws_bwd, self.ws_bwd_bytes,
                                       stream=stream)
            L.moe_expert_up_backward(t["x"], None, self.s_offsets, 1, T, d, fs, self.dtype,
                                     t["Ws_gate"], t["Ws_up"], self.s_dhu, g["dx"], 1,
                                     g["dWs_gate"], g["dWs_up"], self.ws_bwd, self.ws_bwd_bytes,
                                     stream=stream)
            if gated:
                L.moe_linear_backward(t["x"], self.w_s_col, self.dgl, T, d, 1, self.dtype,
                                      g["dw_s"], None, g["dx"], self.ws_lin1, self.ws_lin1_bytes,
                                      stream=stream)
        mk("shared_bwd")
        return g
