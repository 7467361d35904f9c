"""Seeded synthetic inputs for the MoE expert layer.

This module only *draws* tensors; it holds none of the layer's arithmetic.
Both the HIP path and the fp64 CPU oracle consume exactly the tensors it
returns (the oracle upcasts them exactly to float64), so the two sides never
see different numbers.

Workload shapes follow the model families the pages name as MoE workloads:
Mixtral-8x7B and Qwen2-MoE (COMET page, "COMET's Performance"), DeepSeek-MoE
(DisagMoE page, section 4 "Resultados Experimentais").  The pages print no
weights and no dataset for them, so every tensor is a seeded Gaussian:

* "N(0, s)" means variance s (std = sqrt(s)).  Under the std reading the
  router logits collapse to ~0 and the skewed config's bias would send
  50/50 of assignments to experts 0 and 1, contradicting its "about 40%"
  for expert 0; the variance reading gives ~46%.
* fan_in init: W_r, W_gate, W_up, shared gate/up and w_s use 1/d; W_down
  uses 1/f.
* Floating inputs are drawn in float32 and rounded to bfloat16 with
  round-to-nearest-even (the fp32 tiny config stays float32).
* The skewed config's per-expert logit bias is b_e = 1.5*ln((e+1)^-1.2)
  = -1.8*ln(e+1) (natural log), stored as float32.

Two generator back-ends exist, selected by the ``device`` argument: numpy's
PCG64 (host) and torch's device generator (fast at full size on a GPU).
They give different values for the same seed; any one comparison always uses
one draw for both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape and routing options of one synthetic MoE expert layer."""

    name: str
    cfg_id: int
    T: int          # tokens
    d: int          # model dim
    f: int          # expert FFN dim
    E: int          # routed experts
    k: int          # top-k
    renorm: bool    # renormalise the k selected softmax weights
    dtype: str      # "bf16" or "f32" storage of x and weights
    biased: bool = False       # per-expert logit bias (skewed load)
    bias_scale: float = 1.0    # strength of that bias (the skew sweep's axis)
    n_shared: int = 0          # always-on shared SwiGLU experts
    f_shared: int = 0          # their FFN dim
    shared_gated: bool = False # shared output scaled by sigmoid(x . w_s)

    @property
    def R(self) -> int:
        return self.T * self.k

    def flops(self) -> int:
        """Algorithmic flops of one layer forward (no padding, SiLU/softmax ignored)."""
        fl = 2 * self.T * self.d * self.E + 6 * self.T * self.k * self.d * self.f
        fl += self.n_shared * 6 * self.T * self.d * self.f_shared
        if self.shared_gated:
            fl += 2 * self.T * self.d
        return fl

    def shrink(self, T: int, d: int, f: int, f_shared: Optional[int] = None) -> "LayerConfig":
        """Same E, k, score rule, bias and shared experts, smaller T, d, f."""
        return dataclasses.replace(
            self, name=f"{self.name}-small", T=T, d=d, f=f,
            f_shared=(f_shared if f_shared is not None else (f if self.n_shared else 0)))


CONFIGS = {
    "tiny": LayerConfig("tiny", 0, T=128, d=64, f=128, E=4, k=2, renorm=True, dtype="f32"),
    "mixtral": LayerConfig("mixtral", 1, T=4096, d=4096, f=14336, E=8, k=2, renorm=True,
                           dtype="bf16"),
    "qwen2moe": LayerConfig("qwen2moe", 2, T=8192, d=3584, f=2560, E=64, k=8, renorm=True,
                            dtype="bf16", n_shared=1, f_shared=20480, shared_gated=True),
    "mixtral_skew": LayerConfig("mixtral_skew", 3, T=16384, d=4096, f=14336, E=8, k=2,
                                renorm=True, dtype="bf16", biased=True),
    "deepseek": LayerConfig("deepseek", 4, T=32768, d=2048, f=1408, E=64, k=6, renorm=False,
                            dtype="bf16", n_shared=2, f_shared=1408),
}

# The two robustness axes the COMET page reports on ("COMET's Performance":
# speedups across input token lengths, and behaviour under imbalanced expert
# loads), as sweeps of the Mixtral-shape layer: the token count from 128 to
# 32768, and the strength of the skewed workload's router bias from 0 (no
# skew) to twice the stated bias.
SWEEP_TOKENS = (128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768)
SWEEP_BIAS_SCALES = (0.0, 0.5, 1.0, 1.5, 2.0)


def sweep_configs(kind: str):
    """The layers of one sweep: kind "tokens" or "skew"."""
    if kind == "tokens":
        return [dataclasses.replace(CONFIGS["mixtral"], name=f"mixtral_T{T}", T=T)
                for T in SWEEP_TOKENS]
    if kind == "skew":
        return [dataclasses.replace(CONFIGS["mixtral_skew"], name=f"mixtral_skew_b{s:g}",
                                    bias_scale=s) for s in SWEEP_BIAS_SCALES]
    raise ValueError(f"unknown sweep {kind!r} (tokens or skew)")


# tensor ids inside one config's seed space
_TID = {"x": 0, "W_r": 1, "W_gate": 2, "W_up": 3, "W_down": 4, "w_s": 5}


def _shared_tid(s: int, which: str) -> int:
    return 16 + 3 * s + {"gate": 0, "up": 1, "down": 2}[which]


def skew_bias(E: int, scale: float = 1.0) -> np.ndarray:
    """Per-expert router bias of the skewed-load workload (times ``scale``), float32."""
    return np.array([scale * 1.5 * math.log((e + 1) ** -1.2) for e in range(E)],
                    dtype=np.float32)


def _draw_numpy(cfg_id: int, tid: int, seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([seed, cfg_id, tid]))
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def _draw(cfg: LayerConfig, name: str, tid: int, seed: int, shape, std: float, device):
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    if device is None or str(device) == "cpu":
        a = torch.from_numpy(_draw_numpy(cfg.cfg_id, tid, seed, shape, std))
        return a.to(dt)  # torch's float32 -> bfloat16 cast rounds to nearest even
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + cfg.cfg_id * 1009 + tid) & 0x7FFFFFFFFFFFFFFF)
    a = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    a.mul_(std)
    return a.to(dt)


ROUTER_PARTS = ("x", "W_r", "b")


def make_layer(cfg: LayerConfig, seed: int = 0, device=None, T: Optional[int] = None,
               parts=None):
    """Draw every tensor of ``cfg``.

    Returns a dict of torch tensors on ``device`` (host when None):
    x[T,d], W_r[d,E], b[E] (float32, or None), W_gate/W_up[E,d,f], W_down[E,f,d],
    and, for shared experts, Ws_gate/Ws_up[d, n_shared*f_s] (shared expert s
    in columns s*f_s .. (s+1)*f_s - 1: the experts side by side, as one FFN
    of width n_shared*f_s), Ws_down[n_shared,f_s,d], w_s[d] (gated config
    only).  ``T`` overrides the token count (a
    differently sized x, used for bounded samples; on the host back-end its
    rows are the first rows of the full draw).  ``parts``
    restricts the draw to the named tensors (e.g. ``ROUTER_PARTS``); every
    tensor has its own seed, so a partial draw equals the full one.
    """
    import torch
    T = cfg.T if T is None else T
    d, f, E = cfg.d, cfg.f, cfg.E
    want = (lambda n: True) if parts is None else (lambda n: n in parts)
    out = {}
    if want("x"):
        out["x"] = _draw(cfg, "x", _TID["x"], seed, (T, d), 1.0, device)
    if want("W_r"):
        out["W_r"] = _draw(cfg, "W_r", _TID["W_r"], seed, (d, E), 1.0 / math.sqrt(d), device)
    if want("W_gate"):
        out["W_gate"] = _draw(cfg, "W_gate", _TID["W_gate"], seed, (E, d, f), 1.0 / math.sqrt(d), device)
    if want("W_up"):
        out["W_up"] = _draw(cfg, "W_up", _TID["W_up"], seed, (E, d, f), 1.0 / math.sqrt(d), device)
    if want("W_down"):
        out["W_down"] = _draw(cfg, "W_down", _TID["W_down"], seed, (E, f, d), 1.0 / math.sqrt(f), device)
    if want("b"):
        out["b"] = None
        if cfg.biased:
            b = torch.from_numpy(skew_bias(E, cfg.bias_scale))
            out["b"] = b if device is None else b.to(device)
    if cfg.n_shared and want("Ws"):
        fs = cfg.f_shared
        gs, us, ds = [], [], []
        for s in range(cfg.n_shared):
            gs.append(_draw(cfg, "Ws_gate", _shared_tid(s, "gate"), seed, (d, fs), 1.0 / math.sqrt(d), device))
            us.append(_draw(cfg, "Ws_up", _shared_tid(s, "up"), seed, (d, fs), 1.0 / math.sqrt(d), device))
            ds.append(_draw(cfg, "Ws_down", _shared_tid(s, "down"), seed, (fs, d), 1.0 / math.sqrt(fs), device))
        out["Ws_gate"] = torch.cat(gs, dim=1)
        out["Ws_up"] = torch.cat(us, dim=1)
        out["Ws_down"] = torch.stack(ds)
    if want("w_s"):
        out["w_s"] = None
    if cfg.shared_gated and want("w_s"):
        out["w_s"] = _draw(cfg, "w_s", _TID["w_s"], seed, (d,), 1.0 / math.sqrt(d), device)
    return out


def to_f64(layer: dict) -> dict:
    """Exact upcast of every tensor to a float64 numpy array (None stays None)."""
    import torch
    res = {}
    for k, v in layer.items():
        res[k] = None if v is None else v.detach().to("cpu", torch.float64).numpy()
    return res
