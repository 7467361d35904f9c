"""Drive one MoE expert-layer forward through the C ABI.

Allocates the buffers of the path once (torch is used for device memory and
the stream only) and issues the C-ABI calls in order:

    moe_route -> moe_permute -> [shared experts] -> moe_expert_up
              -> moe_expert_down (+ fused combine, or moe_combine)

Two variants of the same layer:

* ``fused=True`` (the fast path): the gather of token rows happens inside
  the layer-0 GEMM's loads (no permuted copy of x), and the combine happens
  inside the layer-1 GEMM's epilogue with fp32 atomic adds into y, which is
  first set to the shared-expert term (or cleared).
* ``fused=False`` (deterministic): x_perm is materialised, the layer-1 GEMM
  writes y_perm, and moe_combine sums the k slots in order.

Shared experts: the ungated ones run as one grouped FFN with E = n_shared
whose rows all read x (row r of shared expert s reads token r - s*T); on the
fused path they add straight into y, on the deterministic path their outputs
are summed into y in expert order by moe_combine.  The gated one writes its
output to a buffer, scaled per token by sigmoid(x . w_s) inside moe_combine,
the gate logit coming from moe_route with E = 1.
"""
from __future__ import annotations

import torch

from . import _lib as L
from .inputs import LayerConfig


class MoeLayer:
    def __init__(self, cfg: LayerConfig, layer: dict, fused: bool = True, keep_logits: bool = True):
        self.cfg = cfg
        self.t = layer
        self.fused = fused
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
        self.x_perm = None if fused else e(R, d, dt=act)
        self.a = e(R, f, dt=act)
        self.y_perm = None if fused else e(R, d)
        self.y = e(T, d)
        self.ws_route_bytes = L.moe_route_workspace_size(d, E, self.dtype)
        self.ws_route = e(max(self.ws_route_bytes, 16), dt=torch.uint8)
        self.ws_perm_bytes = L.moe_permute_workspace_size(T, E, k)
        self.ws_perm = e(max(self.ws_perm_bytes, 16), dt=torch.uint8)
        self.ws_ffn_bytes = L.moe_ffn_workspace_size(E, R, d, f)
        self.ws_ffn = e(max(self.ws_ffn_bytes, 16), dt=torch.uint8)
        # shared experts
        self.ns = cfg.n_shared
        if self.ns:
            fs = cfg.f_shared
            self.s_a = e(self.ns * T, fs, dt=act)
            ar = torch.arange(T, dtype=i32, device=dev)
            self.s_rows = ar.repeat(self.ns).contiguous()
            self.s_offsets = (torch.arange(self.ns + 1, dtype=i32, device=dev) * T).contiguous()
            self.s_ws_bytes = L.moe_ffn_workspace_size(self.ns, self.ns * T, d, fs)
            self.s_ws = e(max(self.s_ws_bytes, 16), dt=torch.uint8)
            if not cfg.shared_gated and not fused:
                self.ys_all = e(self.ns * T, d)
            if cfg.shared_gated:
                self.ys = e(T, d)
                self.g_idx = e(T, 1, dt=i32)
                self.g_w = e(T, 1)
                self.g_logit = e(T, 1)
                self.w_s_col = layer["w_s"].reshape(d, 1).contiguous()
                self.g_ws_bytes = L.moe_route_workspace_size(d, 1, self.dtype)
                self.g_ws = e(max(self.g_ws_bytes, 16), dt=torch.uint8)

    # -- stages ------------------------------------------------------------
    def route(self, stream=None):
        c, t = self.cfg, self.t
        score = L.MOE_SOFTMAX_TOPK_RENORM if c.renorm else L.MOE_SOFTMAX_TOPK
        L.moe_route(t["x"], t["W_r"], t.get("b"), c.T, c.d, c.E, c.k, score, self.dtype,
                    self.idx, self.w, self.logits, self.ws_route, self.ws_route_bytes,
                    stream=stream)

    def permute(self, stream=None):
        c, t = self.cfg, self.t
        L.moe_permute(self.idx, self.w, t["x"], c.T, c.d, c.E, c.k, self.dtype, self.counts,
                      self.offsets, self.perm_token, self.inv, self.perm_w, self.x_perm,
                      self.ws_perm, self.ws_perm_bytes, stream=stream)

    def shared(self, stream=None):
        """Initialise y with the shared-expert term (or clear it when there is
        none and the combine is fused)."""
        c, t = self.cfg, self.t
        if not self.ns:
            if self.fused:
                L.moe_combine(None, None, None, c.T, c.d, c.k, None, None, 0, self.y,
                              stream=stream)
            return
        T, d, fs = c.T, c.d, c.f_shared
        rows = self.ns * T
        if c.shared_gated:
            # gate logit x . w_s (a one-column router), then y = g * S(x) (+ routed later)
            L.moe_route(t["x"], self.w_s_col, None, T, d, 1, 1, L.MOE_SOFTMAX_TOPK, self.dtype,
                        self.g_idx, self.g_w, self.g_logit, self.g_ws, self.g_ws_bytes,
                        stream=stream)
            L.moe_expert_up(t["x"], self.s_rows, self.s_offsets, self.ns, rows, d, fs, self.dtype,
                            t["Ws_gate"], t["Ws_up"], self.s_a, self.s_ws, self.s_ws_bytes,
                            stream=stream)
            L.moe_expert_down(self.s_a, self.s_offsets, self.ns, rows, fs, d, self.dtype,
                              t["Ws_down"], self.ys, None, None, None, self.s_ws, self.s_ws_bytes,
                              stream=stream)
            if self.fused:
                L.moe_combine(None, None, None, T, d, c.k, self.ys, self.g_logit, 0, self.y,
                              stream=stream)
        else:
            L.moe_expert_up(t["x"], self.s_rows, self.s_offsets, self.ns, rows, d, fs, self.dtype,
                            t["Ws_gate"], t["Ws_up"], self.s_a, self.s_ws, self.s_ws_bytes,
                            stream=stream)
            if self.fused:
                # y = 0, then every shared expert adds into it (atomic adds)
                L.moe_combine(None, None, None, T, d, c.k, None, None, 0, self.y, stream=stream)
                L.moe_expert_down(self.s_a, self.s_offsets, self.ns, rows, fs, d, self.dtype,
                                  t["Ws_down"], None, self.s_rows, None, self.y, self.s_ws,
                                  self.s_ws_bytes, stream=stream)
            else:
                # deterministic: per-expert outputs, summed into y in expert order
                L.moe_expert_down(self.s_a, self.s_offsets, self.ns, rows, fs, d, self.dtype,
                                  t["Ws_down"], self.ys_all, None, None, None, self.s_ws,
                                  self.s_ws_bytes, stream=stream)
                for s_ in range(self.ns):
                    L.moe_combine(None, None, None, T, d, c.k, self.ys_all[s_ * T:(s_ + 1) * T],
                                  None, 1 if s_ else 0, self.y, stream=stream)

    def expert_up(self, stream=None):
        c, t = self.cfg, self.t
        R = c.T * c.k
        if self.fused:
            L.moe_expert_up(t["x"], self.perm_token, self.offsets, c.E, R, c.d, c.f, self.dtype,
                            t["W_gate"], t["W_up"], self.a, self.ws_ffn, self.ws_ffn_bytes,
                            stream=stream)
        else:
            L.moe_expert_up(self.x_perm, None, self.offsets, c.E, R, c.d, c.f, self.dtype,
                            t["W_gate"], t["W_up"], self.a, self.ws_ffn, self.ws_ffn_bytes,
                            stream=stream)

    def expert_down(self, stream=None):
        c, t = self.cfg, self.t
        R = c.T * c.k
        if self.fused:
            L.moe_expert_down(self.a, self.offsets, c.E, R, c.f, c.d, self.dtype, t["W_down"],
                              None, self.perm_token, self.perm_w, self.y, self.ws_ffn,
                              self.ws_ffn_bytes, stream=stream)
        else:
            L.moe_expert_down(self.a, self.offsets, c.E, R, c.f, c.d, self.dtype, t["W_down"],
                              self.y_perm, None, None, None, self.ws_ffn, self.ws_ffn_bytes,
                              stream=stream)

    def combine(self, stream=None):
        if self.fused:
            return
        c = self.cfg
        ys = self.ys if (self.ns and c.shared_gated) else None
        gl = self.g_logit if (self.ns and c.shared_gated) else None
        acc = 1 if (self.ns and not c.shared_gated) else 0
        L.moe_combine(self.y_perm, self.inv, self.w, c.T, c.d, c.k, ys, gl, acc, self.y,
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
