"""The forward pass captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay, with eager work and synchronisations between them
(new token rows copied into the captured input buffer, the output cleared),
writes the bits an eager forward writes for the same inputs."""
import sys

import pytest
import torch

from mixture_experts_layer_top_amd.inputs import CONFIGS, make_layer

pytestmark = pytest.mark.gpu

CASES = {
    "mixtral_k64": CONFIGS["mixtral"].shrink(T=2000, d=512, f=320),          # compact rows
    "qwen2moe_k64": CONFIGS["qwen2moe"].shrink(T=1024, d=320, f=192, f_shared=448),  # gated shared
    "deepseek": CONFIGS["deepseek"].shrink(T=1500, d=256, f=136, f_shared=136),      # general kernel
    "tiny": CONFIGS["tiny"],                                                 # fp32 kernels
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def L():
    from mixture_experts_layer_top_amd import _lib
    _lib.load()
    return _lib


@pytest.mark.parametrize("path", ["fast", "atomic"])
@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(L, name, path):
    from mixture_experts_layer_top_amd.layer import MoeLayer
    cfg = CASES[name]
    log(f"[graph] {name} path={path} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
    layer = make_layer(cfg, seed=61, device="cuda")
    x1 = layer["x"].clone()
    x2 = make_layer(cfg, seed=62, device="cuda", parts=("x",))["x"]
    want = []
    for x in (x1, x2):
        layer["x"].copy_(x)
        m_e = MoeLayer(cfg, layer, path=path)
        want.append(m_e.forward().clone())
        torch.cuda.synchronize()
    assert not torch.equal(want[0], want[1])
    layer["x"].copy_(x1)
    m = MoeLayer(cfg, layer, path=path)
    g = m.capture_graph()
    for rep in range(6):
        j = rep % 2
        layer["x"].copy_(x2 if j else x1)  # eager work between replays
        m.y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if path == "fast":
            assert torch.equal(m.y, want[j]), rep
        else:  # atomic adds: the order of a token's k adds is not fixed
            r = float(want[j].pow(2).mean().sqrt())
            assert float((m.y - want[j]).abs().max()) <= 1e-5 * r, rep
