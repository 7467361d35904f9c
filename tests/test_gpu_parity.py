"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Bars (the design notes derive each):
* routing: the oracle's selection run on the GPU's own fp32 logits equals
  the GPU's top-k indices bit for bit; the GPU's fp32 logits are within the
  certified fp32 error bound of the fp64 logits, and every token whose fp64
  selection differs from the GPU's is a certified near-tie;
* weights: within a relative bound derived from fp32 exp/sum/divide;
* dispatch: counts, offsets, perm_token, inv, perm_w (and x_perm) equal the
  oracle's on the GPU's selection, bit for bit;
* output: max |y_gpu - y_ref| <= tau * rms(y_ref), tau = 2e-2 for bf16
  inputs with fp32 accumulation and 1e-4 for the fp32 layer, y_ref the fp64
  oracle at the GPU's selection.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mixture_experts_layer_top_amd.inputs import CONFIGS, make_layer, to_f64

pytestmark = pytest.mark.gpu

TAU = {"bf16": 2e-2, "f32": 1e-4}
U32 = 2.0 ** -24

MID = {
    "tiny": CONFIGS["tiny"],
    "mixtral": CONFIGS["mixtral"].shrink(T=2000, d=520, f=392),
    "qwen2moe": CONFIGS["qwen2moe"].shrink(T=1024, d=264, f=200, f_shared=256),
    "mixtral_skew": CONFIGS["mixtral_skew"].shrink(T=3000, d=256, f=256),
    "deepseek": CONFIGS["deepseek"].shrink(T=1500, d=256, f=136, f_shared=136),
    # K a multiple of 64 (the ping-pong GEMM), N ragged against its tiles
    "mixtral_k64": CONFIGS["mixtral"].shrink(T=2000, d=512, f=320),
    "qwen2moe_k64": CONFIGS["qwen2moe"].shrink(T=1024, d=320, f=192, f_shared=448),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def L():
    from mixture_experts_layer_top_amd import _lib
    _lib.load()
    return _lib


def run_layer(cfg, layer, path="fast"):
    from mixture_experts_layer_top_amd.layer import MoeLayer
    if path is True or path is False:
        path = "atomic" if path else "reference"
    m = MoeLayer(cfg, layer, path=path)
    m.forward()
    torch.cuda.synchronize()
    return m


def rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


class LazyExperts:
    """fp64 view of a [E, a, b] device tensor, converted one expert at a time."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        return self.t[e].to("cpu", torch.float64).numpy()


def host_layer(layer, lazy=False):
    out = {}
    for k_, v in layer.items():
        if v is None:
            out[k_] = None
        elif lazy and v.dim() == 3:
            out[k_] = LazyExperts(v)
        else:
            out[k_] = v.to("cpu", torch.float64).numpy()
    return out


def check_routing(cfg, m, h):
    """Checks (i) and (ii) of the routing bar; returns the GPU selection and
    the near-tie tokens."""
    k, E = cfg.k, cfg.E
    L32 = m.logits.to("cpu", torch.float64).numpy()
    idx_g = m.idx.cpu().numpy().astype(np.int64)
    w_g = m.w.cpu().numpy().astype(np.float64)
    # (i) the decision on the GPU's own logits is exact
    idx_o = O.select_topk(L32, k)
    bad = np.nonzero(np.any(idx_o != idx_g, axis=1))[0]
    assert len(bad) == 0, f"selection differs on GPU logits at tokens {bad[:10]}"
    w_o = O.topk_weights(L32, idx_o, cfg.renorm)
    span = float(np.max(L32.max(1) - L32.min(1)))
    w_rtol = (2 * E + 16 + 4 * span) * U32
    np.testing.assert_allclose(w_g, w_o, rtol=w_rtol, atol=0)
    # (ii) against fp64 logits
    L64 = O.router_logits(h["x"], h["W_r"], h.get("b"))
    bound = O.fp32_logit_error_bound(h["x"], h["W_r"], h.get("b"))
    assert np.all(np.abs(L32 - L64) <= bound[:, None]), "fp32 logits outside the certified bound"
    idx64 = O.select_topk(L64, k)
    diff = np.nonzero(np.any(idx64 != idx_g, axis=1))[0]
    margin = O.selection_margin(L64, k)
    assert np.all(margin[diff] <= 2 * bound[diff]), "a routing difference is not a near-tie"
    if len(diff):
        log(f"  near-tie tokens (fp64 selection differs, certified): {diff.tolist()}")
    return idx_g, w_g, diff


def check_dispatch(cfg, m, idx_g, w_g):
    counts, offsets, perm_token, inv, perm_w = O.dispatch(idx_g, w_g, cfg.E)
    assert np.array_equal(m.counts.cpu().numpy(), counts)
    assert np.array_equal(m.offsets.cpu().numpy(), offsets)
    assert np.array_equal(m.perm_token.cpu().numpy(), perm_token)
    assert np.array_equal(m.inv.cpu().numpy(), inv)
    assert np.array_equal(m.perm_w.cpu().numpy().astype(np.float64), perm_w)
    return perm_token


def check_y(cfg, y_g, y_ref, what=""):
    err = float(np.max(np.abs(y_g - y_ref)))
    r = rms(y_ref)
    tau = TAU[cfg.dtype]
    log(f"  {cfg.name} {what}: max|dy| / rms = {err / r:.3e} (bar {tau:g})")
    assert err <= tau * r


# ---------------------------------------------------------------- mid sizes


PATH_IDS = ["fast", "fast32", "atomic", "reference"]


@pytest.mark.parametrize("path", PATH_IDS)
@pytest.mark.parametrize("name", list(MID))
def test_layer_parity_mid(L, name, path):
    cfg = MID[name]
    log(f"[parity-mid] {name} path={path} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
    layer = make_layer(cfg, seed=11, device="cuda")
    m = run_layer(cfg, layer, path)
    h = host_layer(layer)
    idx_g, w_g, _ = check_routing(cfg, m, h)
    perm_token = check_dispatch(cfg, m, idx_g, w_g)
    if path == "reference":
        assert torch.equal(m.x_perm.cpu(), layer["x"].cpu()[torch.from_numpy(perm_token)])
    ref = O.forward(h, cfg.k, cfg.renorm, idx=idx_g)
    check_y(cfg, m.y.cpu().double().numpy(), ref["y"], path)


@pytest.mark.parametrize("path", ["fast", "reference"])
@pytest.mark.parametrize("name", ["deepseek", "qwen2moe"])
def test_deterministic_paths_are_bitwise_repeatable(L, name, path):
    cfg = MID[name]
    layer = make_layer(cfg, seed=3, device="cuda")
    m1 = run_layer(cfg, layer, path)
    y1, p1 = m1.y.clone(), m1.perm_token.clone()
    m2 = run_layer(cfg, layer, path)
    assert torch.equal(m2.perm_token, p1)
    assert torch.equal(m2.y, y1)


@pytest.mark.parametrize("name", ["qwen2moe", "qwen2moe_k64"])
def test_paths_agree(L, name):
    """fp32 rows: the same products whichever path; only the order of the fp32
    adds may differ (atomic), and fast32 and reference add in the same order.
    Compact rows (the fast path where d is a multiple of 32, else fast32's):
    each term moves by at most 2^-11 of its segment's largest magnitude, so
    |y_fast - y_ref| <= 2^-11 (max |y_perm| sum_j w_j + g max |y_shared|)."""
    cfg = MID[name]
    layer = make_layer(cfg, seed=5, device="cuda")
    ms = {p: run_layer(cfg, layer, p) for p in PATH_IDS}
    ys = {p: m.y.cpu().double().numpy() for p, m in ms.items()}
    b = ys["reference"]
    for p in ("fast32", "atomic"):
        assert np.max(np.abs(ys[p] - b)) <= 1e-5 * rms(b), p
    assert np.array_equal(ys["fast32"], ys["reference"])  # identical sums in identical order
    m32 = ms["fast32"]
    wsum = m32.w.sum(dim=1).max().item()
    bound = float(m32.y_perm.abs().max()) * wsum
    if cfg.n_shared:
        bound += float(m32.ys.abs().max())  # the gate is at most 1
    assert ms["fast"].comb == ("separate16" if cfg.d % 32 == 0 else "separate")
    assert np.max(np.abs(ys["fast"] - b)) <= 2.0 ** -11 * bound * (1 + 1e-6) + 1e-5 * rms(b)


def restore(y_h, y_s):
    """Values of compact rows: y_h[r, c] * y_s[r, c / 32] (exact in fp32)."""
    return y_h.float() * y_s.repeat_interleave(32, dim=1)


@pytest.mark.parametrize("name", ["deepseek", "qwen2moe_k64", "mixtral_skew", "mixtral_k64"])
def test_compact_rows_encode_the_fp32_rows(L, name):
    """The compact layer-1 rows against the fp32 rows of the same GEMM (same
    tiles, same accumulation order, so the same fp32 values), routed and
    shared: every factor is a power of two that puts the segment's largest
    magnitude in [2^14, 2^15) (2^-126 for segments below 2^-112), every fp16
    value is the fp32 value over the factor rounded to nearest even, bit for
    bit; and the combine over the compact rows writes the bits moe_combine
    writes over the restored rows."""
    cfg = MID[name]
    log(f"[compact] encode {name} T={cfg.T} d={cfg.d} f={cfg.f}")
    layer = make_layer(cfg, seed=21, device="cuda")
    m32 = run_layer(cfg, layer, "fast32")
    m16 = run_layer(cfg, layer, "fast")
    assert m16.comb == "separate16" and m32.comb == "separate"
    pairs = [(m32.y_perm, m16.y_h, m16.y_s)]
    if cfg.n_shared:
        pairs.append((m32.ys, m16.ys_h, m16.ys_s))
    for y32, yh, ysc in pairs:
        R, d = y32.shape
        seg = y32.view(R, d // 32, 32)
        mx = seg.abs().amax(dim=2)
        mant, _ = torch.frexp(ysc)
        assert torch.all(mant == 0.5)
        big = mx >= 2.0 ** -112
        scaled = mx[big] / ysc[big]
        assert torch.all((scaled >= 2.0 ** 14) & (scaled < 2.0 ** 15))
        assert torch.all(ysc[~big] == 2.0 ** -126)
        want = (seg / ysc.unsqueeze(2)).to(torch.float16).view(R, d)
        assert torch.equal(yh.view(torch.int16), want.view(torch.int16))
    T, d, k = cfg.T, cfg.d, cfg.k
    ys = restore(m16.ys_h, m16.ys_s).contiguous() if cfg.n_shared else None
    gl = m16.g_logit if (cfg.n_shared and cfg.shared_gated) else None
    y = torch.empty_like(m16.y)
    L.moe_combine(restore(m16.y_h, m16.y_s).contiguous(), m16.inv, m16.w, T, d, k, ys, gl, 0, y)
    torch.cuda.synchronize()
    assert torch.equal(y, m16.y)


@pytest.mark.parametrize("scale_log2", [24, -30])
def test_compact_rows_far_outside_fp16_range(L, scale_log2):
    """W_down and the shared experts' W_down scaled by 2^24 and by 2^-30 (exact
    in bf16): layer-1 outputs far above fp16's largest value, or below its
    smallest, are kept by the segment factors, and y stays within the bar of
    the oracle on the scaled layer."""
    cfg = MID["deepseek"]
    log(f"[compact] range 2^{scale_log2}")
    layer = make_layer(cfg, seed=23, device="cuda")
    s = 2.0 ** scale_log2
    layer["W_down"] = (layer["W_down"] * s).contiguous()
    layer["Ws_down"] = (layer["Ws_down"] * s).contiguous()
    m = run_layer(cfg, layer, "fast")
    assert m.comb == "separate16"
    h = host_layer(layer)
    idx_g, w_g, _ = check_routing(cfg, m, h)
    check_y(cfg, m.y.cpu().double().numpy(), O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"],
            f"compact 2^{scale_log2}")


# ---------------------------------------------------------------- edge cases


def small_cfg(**kw):
    base = dict(name="edge", cfg_id=9, T=130, d=72, f=40, E=8, k=2, renorm=True, dtype="bf16")
    base.update(kw)
    return CONFIGS["mixtral"].__class__(**base)


@pytest.mark.parametrize("T,f", [(1, 40), (65, 40), (257, 64), (130, 64), (63, 128)])
def test_compact_rows_ragged(L, T, f):
    """d = 96 (three 32-column segments, a partial column tile) on the fast
    path: compact rows from the general kernel (f = 40, K not a multiple of
    64) and from the ping-pong kernel (f = 64, 128), ragged token counts."""
    cfg = small_cfg(T=T, d=96, f=f)
    log(f"[compact] ragged T={T} d=96 f={f}")
    layer = make_layer(cfg, seed=40 + T, device="cuda")
    m = run_layer(cfg, layer, "fast")
    assert m.comb == "separate16"
    h = host_layer(layer)
    idx_g, w_g, _ = check_routing(cfg, m, h)
    check_dispatch(cfg, m, idx_g, w_g)
    check_y(cfg, m.y.cpu().double().numpy(), O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"])


@pytest.mark.parametrize("T", [1, 63, 65, 257])
def test_ragged_token_counts(L, T):
    cfg = small_cfg(T=T)
    log(f"[edge] ragged T={T}")
    layer = make_layer(cfg, seed=T, device="cuda")
    m = run_layer(cfg, layer, "fast")
    h = host_layer(layer)
    idx_g, w_g, _ = check_routing(cfg, m, h)
    check_dispatch(cfg, m, idx_g, w_g)
    check_y(cfg, m.y.cpu().double().numpy(), O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"])


@pytest.mark.parametrize("E,k", [(1, 1), (4, 4), (256, 8), (3, 2), (8, 1), (64, 1), (16, 16),
                                 (64, 20), (256, 256)])
def test_expert_count_extremes(L, E, k):
    """Expert and slot counts at the ends of the accepted range: one expert,
    top-1 over 8 and 64 (renormalised weights exactly 1), k = E = 16 (the
    last k whose picks stay one per lane of the router's 16-lane row),
    k = 20 > 16 (picks written one by one), k = E = 256 (every token on every
    expert; the combine's run-time slot loop)."""
    cfg = small_cfg(E=E, k=k, T=300, d=64, f=48)
    log(f"[edge] E={E} k={k}")
    layer = make_layer(cfg, seed=E, device="cuda")
    m = run_layer(cfg, layer, "fast")
    h = host_layer(layer)
    idx_g, w_g, _ = check_routing(cfg, m, h)
    check_dispatch(cfg, m, idx_g, w_g)
    check_y(cfg, m.y.cpu().double().numpy(), O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"])
    if k == 1 and cfg.renorm:
        assert np.all(w_g == 1.0)


@pytest.mark.parametrize("nk", [1, 2, 3, 5])
def test_gemm_stage_counts(L, nk):
    """d = f = 64 nk: the ping-pong GEMM with 1, 2, 3 and 5 K stages (its
    prologue and ring take different branches for nk < 3)."""
    cfg = small_cfg(E=16, k=4, T=700, d=64 * nk, f=64 * nk)
    log(f"[edge] GEMM stages nk={nk}")
    layer = make_layer(cfg, seed=40 + nk, device="cuda")
    for path in PATH_IDS:
        m = run_layer(cfg, layer, path)
        h = host_layer(layer)
        idx_g, w_g, _ = check_routing(cfg, m, h)
        check_dispatch(cfg, m, idx_g, w_g)
        check_y(cfg, m.y.cpu().double().numpy(), O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"],
                path)


def test_gemm_tail_split_and_unsplit_agree(L):
    """The FFN workspace enables the tail split (K split of the last round's
    tiles, partials summed in a fixed order by a second pass).  Without it
    the GEMMs run unsplit.  Both meet the bar, each is bitwise repeatable,
    and they agree to within a quarter of the bar."""
    cfg = MID["mixtral_k64"]  # 48 layer-0 tiles: a mostly idle single round
    layer = make_layer(cfg, seed=21, device="cuda")
    from mixture_experts_layer_top_amd.layer import MoeLayer
    ys = {}
    for mode in ("split", "unsplit"):
        outs = []
        for _ in range(2):
            m = MoeLayer(cfg, layer, path="fast")
            if mode == "unsplit":
                m.ws_ffn = torch.empty(16, dtype=torch.uint8, device="cuda")
                m.ws_ffn_bytes = 16
            m.forward()
            torch.cuda.synchronize()
            outs.append(m.y.clone())
        assert torch.equal(outs[0], outs[1]), mode
        ys[mode] = outs[0].cpu().double().numpy()
    h = host_layer(layer)
    idx_g = m.idx.cpu().numpy().astype(np.int64)
    ref = O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"]
    for mode, y in ys.items():
        check_y(cfg, y, ref, mode)
    # a different fp32 summation grouping in layer 0 can move a bf16-rounded
    # SwiGLU output by one ulp (2^-8 relative), so the two differ by far more
    # than fp32 rounding, but stay well inside the bar
    assert np.max(np.abs(ys["split"] - ys["unsplit"])) <= TAU[cfg.dtype] / 4 * rms(ref)


def test_empty_experts(L):
    cfg = small_cfg(E=8, k=2, T=500, biased=True)
    layer = make_layer(cfg, seed=1, device="cuda")
    layer["b"] = torch.tensor([0, -1e4, 0, -1e4, 0, 0, -1e4, 0], dtype=torch.float32,
                              device="cuda")
    m = run_layer(cfg, layer, "fast")
    counts = m.counts.cpu().numpy()
    assert counts[1] == counts[3] == counts[6] == 0
    h = host_layer(layer)
    idx_g, w_g, _ = check_routing(cfg, m, h)
    check_dispatch(cfg, m, idx_g, w_g)
    check_y(cfg, m.y.cpu().double().numpy(), O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"])


def test_exact_ties_go_to_lower_index(L):
    cfg = small_cfg(E=8, k=3, T=256)
    layer = make_layer(cfg, seed=2, device="cuda")
    layer["W_r"][:, 6] = layer["W_r"][:, 1]
    layer["W_r"][:, 7] = layer["W_r"][:, 1]
    m = run_layer(cfg, layer, "fast")
    L32 = m.logits.cpu().numpy()
    assert np.array_equal(L32[:, 6], L32[:, 1]) and np.array_equal(L32[:, 7], L32[:, 1])
    idx = m.idx.cpu().numpy()
    for row in idx:
        r = list(row)
        for hi in (6, 7):
            if hi in r:
                assert 1 in r and r.index(1) < r.index(hi)
        if 7 in r:
            assert 6 in r and r.index(6) < r.index(7)


@pytest.mark.parametrize("name", ["mixtral", "deepseek", "mixtral_skew"])
def test_zero_token_closed_form(L, name):
    cfg = MID[name]
    layer = make_layer(cfg, seed=4, device="cuda")
    layer["x"][5].zero_()
    m = run_layer(cfg, layer, "fast")
    idx = m.idx[5].cpu().numpy()
    w = m.w[5].cpu().double().numpy()
    if cfg.biased:
        q = 2.0 ** -1.8
        assert idx.tolist() == [0, 1]
        np.testing.assert_allclose(w, [1 / (1 + q), q / (1 + q)], rtol=1e-6)
    else:
        assert idx.tolist() == list(range(cfg.k))
        np.testing.assert_allclose(w, 1.0 / (cfg.k if cfg.renorm else cfg.E), rtol=1e-6)


def test_zero_tokens_is_noop(L):
    cfg = small_cfg(T=0)
    layer = make_layer(cfg, seed=0, device="cuda")
    from mixture_experts_layer_top_amd.layer import MoeLayer
    m = MoeLayer(cfg, layer, path="fast")
    m.counts.fill_(7)
    m.offsets.fill_(7)
    m.forward()
    torch.cuda.synchronize()
    assert m.counts.cpu().tolist() == [0] * cfg.E
    assert m.offsets.cpu().tolist() == [0] * (cfg.E + 1)


def test_zero_projection_exact_zero(L):
    cfg = MID["mixtral"]
    layer = make_layer(cfg, seed=6, device="cuda")
    layer["W_up"].zero_()
    m = run_layer(cfg, layer, "fast")
    assert torch.count_nonzero(m.y).item() == 0


def test_down_projection_homogeneity(L):
    cfg = MID["deepseek"]
    layer = make_layer(cfg, seed=7, device="cuda")
    y1 = run_layer(cfg, layer, "reference").y.clone()
    layer["W_down"].mul_(2)
    layer["Ws_down"].mul_(2)
    y2 = run_layer(cfg, layer, "reference").y
    assert torch.equal(y2, 2 * y1)


# ---------------------------------------------------------------- full sizes


def check_full_sampled(cfg, n_sample=24):
    """The layer at full size, in the launch configuration the benchmark
    times (the "fast" path): routing and dispatch checked on every token, y on
    a sample of tokens the oracle computes one expert group at a time.
    Returns the GPU's per-expert counts."""
    log(f"[full] {cfg.name} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
    layer = make_layer(cfg, seed=0, device="cuda")
    m = run_layer(cfg, layer, "fast")
    h = host_layer(layer, lazy=True)
    idx_g, w_g, near = check_routing(cfg, m, h)
    log("  routing ok")
    check_dispatch(cfg, m, idx_g, w_g)
    log("  dispatch ok")
    counts = m.counts.cpu().numpy()
    rng = np.random.default_rng(123)
    ts = set([0, cfg.T - 1]) | set(rng.choice(cfg.T, min(n_sample, cfg.T), replace=False).tolist())
    small_e = int(np.argmin(counts))
    ts |= set(np.nonzero(np.any(idx_g == small_e, axis=1))[0][:4].tolist())
    ts |= set(near.tolist())
    ts = np.array(sorted(ts))
    sub = dict(h, x=h["x"][ts])
    ref = O.forward(sub, cfg.k, cfg.renorm, idx=idx_g[ts])
    check_y(cfg, m.y.cpu().double().numpy()[ts], ref["y"], f"{len(ts)} sampled tokens")
    return counts


def test_layer1_operand_above_4GiB(L):
    """Layer 1's A operand beyond 4 GiB (T = 133120 tokens, f = 8192: 266240
    x 8192 bf16 = 4.36e9 bytes), past the ping-pong kernel's 32-bit operand
    offsets: layer 1 runs on the general kernel (64-bit addressing), layer 0
    on the ping-pong kernel (x is 1.1 GB). Routing and dispatch on every
    token, y on sampled tokens, through the benchmark's launch path."""
    cfg = dataclasses.replace(CONFIGS["mixtral"], name="mixtral_bigA", T=133120, f=8192)
    assert cfg.T * cfg.k * cfg.f * 2 > 2 ** 32 > cfg.T * cfg.d * 2
    check_full_sampled(cfg, n_sample=16)
    torch.cuda.empty_cache()


def check_full(cfg):
    """The layer at full size in the launch configuration the benchmark times
    (the "fast" path): routing and dispatch on every token, and y compared
    on all T x d elements with the oracle at the GPU's selection (experts
    converted to float64 one at a time)."""
    log(f"[full] {cfg.name} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k} (every token)")
    layer = make_layer(cfg, seed=0, device="cuda")
    m = run_layer(cfg, layer, "fast")
    h = host_layer(layer, lazy=True)
    idx_g, w_g, near = check_routing(cfg, m, h)
    log(f"  routing ok ({len(near)} certified near-ties)")
    check_dispatch(cfg, m, idx_g, w_g)
    log("  dispatch ok")
    y = m.y.cpu().double().numpy()
    del m, layer
    torch.cuda.empty_cache()
    ref = O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"]
    check_y(cfg, y, ref, "all tokens")


@pytest.mark.parametrize("name", ["tiny", "mixtral", "qwen2moe", "mixtral_skew", "deepseek"])
def test_full_size_every_token(L, name):
    check_full(CONFIGS[name])


def test_permute_large_histogram_path(L):
    """256 experts and more than 32768 / 256 blocks of 256 tokens: the
    permute takes its separate-scan path (block histograms with atomic
    totals, one scan workgroup, then the ranks from the scanned bases).
    f = 512: with a very narrow FFN (f = 48) the bf16 rounding of the
    layer-0 output alone moves some of the 2.1M outputs by 2.7e-2 rms (CPU
    emulation), past the bar that the workloads' widths keep well inside."""
    cfg = small_cfg(E=256, k=8, T=33001, d=64, f=512)
    log(f"[edge] permute scan path T={cfg.T} E={cfg.E} k={cfg.k}")
    layer = make_layer(cfg, seed=8, device="cuda")
    for path in ("fast", "reference"):
        m = run_layer(cfg, layer, path)
        h = host_layer(layer)
        idx_g, w_g, _ = check_routing(cfg, m, h)
        perm_token = check_dispatch(cfg, m, idx_g, w_g)
        if path == "reference":
            assert torch.equal(m.x_perm.cpu(), layer["x"].cpu()[torch.from_numpy(perm_token)])
        check_y(cfg, m.y.cpu().double().numpy(),
                O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"], path)


@pytest.mark.parametrize("d", [72, 96])
@pytest.mark.parametrize("path", ["fast", "reference"])
def test_combine_more_than_eight_slots(L, path, d):
    """k = 10 of 16 experts: the combine's run-time slot loop (d = 96: over
    compact rows on the fast path)."""
    cfg = small_cfg(E=16, k=10, T=600, d=d, f=40)
    log(f"[edge] combine k={cfg.k} d={d} path={path}")
    layer = make_layer(cfg, seed=10, device="cuda")
    m = run_layer(cfg, layer, path)
    h = host_layer(layer)
    idx_g, w_g, _ = check_routing(cfg, m, h)
    check_dispatch(cfg, m, idx_g, w_g)
    check_y(cfg, m.y.cpu().double().numpy(), O.forward(h, cfg.k, cfg.renorm, idx=idx_g)["y"], path)


@pytest.mark.parametrize("E,k,T,d", [(8, 2, 16400, 256), (16, 4, 16390, 512), (24, 3, 32770, 128),
                                     (40, 5, 32768, 192), (64, 6, 33000, 64), (64, 4, 32800, 1024),
                                     (64, 8, 9000, 256), (56, 4, 8200, 384)])
def test_route_long_batches(L, E, k, T, d):
    """Batches long enough for the router's shared-W_r kernel (a workgroup
    of 16 tokens per wave on every compute unit) and, at 56 and 64 experts,
    for the 64- and 32-token workgroups of the K-splitting kernel (selection
    with 4 and 8 lanes per token): routing exact on the GPU's logits and
    within the fp32 bound of the fp64 logits, dispatch bit-exact; ragged last
    workgroups (T not a multiple of its tokens)."""
    cfg = small_cfg(E=E, k=k, T=T, d=d, f=64)
    log(f"[edge] long-batch route T={T} d={d} E={E} k={k}")
    layer = make_layer(cfg, seed=30 + E, device="cuda")
    m = run_layer(cfg, layer, "fast")
    h = host_layer(layer)
    idx_g, w_g, _ = check_routing(cfg, m, h)
    check_dispatch(cfg, m, idx_g, w_g)


def test_nan_token_gets_valid_distinct_experts(L):
    """A token whose x row holds a NaN has NaN logits for every expert; the
    selection must still give k distinct experts in [0, E), so the dispatch
    and the gather stay in bounds, and every other token is unaffected."""
    cfg = small_cfg(E=8, k=3, T=300)
    log("[edge] NaN token")
    layer = make_layer(cfg, seed=12, device="cuda")
    layer["x"][7, 5] = float("nan")
    m = run_layer(cfg, layer, "reference")
    idx = m.idx.cpu().numpy()
    assert np.all((idx >= 0) & (idx < cfg.E))
    assert all(len(set(r)) == cfg.k for r in idx.tolist())
    assert idx[7].tolist() == [0, 1, 2]  # all logits NaN: they rank as equal, lower index first
    counts = m.counts.cpu().numpy()
    assert counts.sum() == cfg.T * cfg.k
    h = host_layer(layer)
    ok = np.arange(cfg.T) != 7
    L32 = m.logits.to("cpu", torch.float64).numpy()
    assert np.array_equal(O.select_topk(L32[ok], cfg.k), idx[ok].astype(np.int64))
    idx_g = idx.astype(np.int64)
    w_g = m.w.cpu().numpy().astype(np.float64)  # token 7's weights are NaN
    counts, offsets, perm_token, inv, perm_w = O.dispatch(idx_g, w_g, cfg.E)
    assert np.array_equal(m.counts.cpu().numpy(), counts)
    assert np.array_equal(m.offsets.cpu().numpy(), offsets)
    assert np.array_equal(m.perm_token.cpu().numpy(), perm_token)
    assert np.array_equal(m.inv.cpu().numpy(), inv)
    assert np.array_equal(m.perm_w.cpu().numpy().astype(np.float64), perm_w, equal_nan=True)
    x_ref = layer["x"].cpu()[torch.from_numpy(perm_token)]
    assert torch.equal(torch.nan_to_num(m.x_perm.cpu(), nan=7.0), torch.nan_to_num(x_ref, nan=7.0))
    y = m.y.cpu().double().numpy()
    assert np.all(np.isfinite(np.delete(y, 7, axis=0)))
    sub = dict(h, x=h["x"][ok])
    ref = O.forward(sub, cfg.k, cfg.renorm, idx=idx_g[ok])["y"]
    check_y(cfg, y[ok], ref, "tokens without NaN")


# ---------------------------------------------------------------- sweeps


@pytest.mark.parametrize("T", [128, 512, 32768])
def test_token_sweep_sampled(L, T):
    """Points of the token-count sweep of the Mixtral-shape layer at full d, f."""
    from mixture_experts_layer_top_amd.inputs import sweep_configs
    cfg = {c.T: c for c in sweep_configs("tokens")}[T]
    counts = check_full_sampled(cfg, n_sample=16)
    assert counts.sum() == cfg.T * cfg.k


@pytest.mark.parametrize("scale", [0.0, 2.0])
def test_skew_sweep_sampled(L, scale):
    """Ends of the router-bias-strength sweep: no skew, and twice the skewed
    workload's bias (expert 0 then sits at the top-2 ceiling of one half of
    the assignments, and the last experts get almost none or none)."""
    from mixture_experts_layer_top_amd.inputs import sweep_configs
    cfg = {c.bias_scale: c for c in sweep_configs("skew")}[scale]
    counts = check_full_sampled(cfg, n_sample=16)
    share = counts / counts.sum()
    if scale == 0.0:
        assert np.all(np.abs(share - 0.125) <= 0.02), share
    else:
        assert 0.48 <= share[0] <= 0.5 and share[7] < 0.01, share


@pytest.mark.parametrize("k", [2, 6, 10])
def test_compact_combine_every_term_combination(L, k):
    """moe_combine_f16 through the C ABI on seeded compact rows (fp16 values,
    power-of-two factors), for every combination of its terms: routed only,
    shared only (gated or not), both, neither (y cleared), with accumulate 0
    and 1; each against moe_combine over the restored rows, bit for bit."""
    T, d, E = 333, 96, 16
    R = T * k
    log(f"[compact] combine terms k={k}")
    g = torch.Generator(device="cpu").manual_seed(50 + k)
    y_h = torch.randn(R, d, generator=g).to(torch.float16).cuda()
    y_s = torch.ldexp(torch.ones(R, d // 32), torch.randint(-30, 30, (R, d // 32), generator=g)).cuda()
    inv = torch.stack([torch.randperm(R, generator=g)[:T] for _ in range(k)], dim=1).to(torch.int32).cuda()
    w = torch.rand(T, k, generator=g).cuda()
    ys_h = torch.randn(T, d, generator=g).to(torch.float16).cuda()
    ys_s = torch.ldexp(torch.ones(T, d // 32), torch.randint(-8, 8, (T, d // 32), generator=g)).cuda()
    gl = torch.randn(T, generator=g).cuda()
    y0 = torch.randn(T, d, generator=g).cuda()
    rows, shared = restore(y_h, y_s).contiguous(), restore(ys_h, ys_s).contiguous()
    for routed in (True, False):
        for sh in ("none", "plain", "gated"):
            for acc in (0, 1):
                y16, y32 = y0.clone(), y0.clone()
                L.moe_combine_f16(y_h if routed else None, y_s if routed else None,
                                  inv if routed else None, w if routed else None, T, d, k,
                                  None if sh == "none" else ys_h, None if sh == "none" else ys_s,
                                  gl if sh == "gated" else None, acc, y16)
                L.moe_combine(rows if routed else None, inv if routed else None,
                              w if routed else None, T, d, k, None if sh == "none" else shared,
                              gl if sh == "gated" else None, acc, y32)
                torch.cuda.synchronize()
                assert torch.equal(y16, y32), (routed, sh, acc)


def test_compact_rows_keep_nan_without_losing_their_segment(L):
    """Column 5 of every W_down set to +inf (bf16 holds it): each expert row's
    column 5 sums infinite terms of both signs, so it is NaN on both paths.
    The compact rows keep the NaN, and the NaN does not set its segment's
    scale: y has the same NaN entries on both paths, and every other entry,
    including columns 0..31 beside it, agrees to the compact rows' bound."""
    cfg = MID["mixtral_k64"]
    log("[compact] NaN column")
    layer = make_layer(cfg, seed=31, device="cuda")
    layer["W_down"][:, :, 5] = float("inf")
    m32 = run_layer(cfg, layer, "fast32")
    m16 = run_layer(cfg, layer, "fast")
    assert m16.comb == "separate16"
    y32, y16 = m32.y, m16.y
    nan32, nan16 = torch.isnan(y32), torch.isnan(y16)
    assert nan32[:, 5].all() and torch.equal(nan32, nan16)
    ok = ~nan32
    assert torch.isfinite(y32[ok]).all() and torch.isfinite(y16[ok]).all()
    yp = m32.y_perm
    fmax = float(torch.where(torch.isfinite(yp), yp.abs(), torch.zeros_like(yp)).amax())
    err = (y16[ok] - y32[ok]).abs()
    assert float(err.max()) <= 2.0 ** -11 * fmax * 1.000001
    # the segment holding the NaN column is as precise as its neighbours
    near = (y16[:, :32] - y32[:, :32]).abs()[ok[:, :32]]
    assert float(near.max()) <= 2.0 ** -11 * fmax * 1.000001


def _wide_pads(counts):
    """Rows to add to each expert so that its last rows exceed half a tile
    (200 of 256): every row of the expert then sits in a whole tile."""
    pads = []
    for c in counts:
        rem = c % 256
        pads.append(200 - rem if 0 < rem <= 128 else 0)
    return pads


@pytest.mark.parametrize("counts,d,f", [
    ([300, 44, 0, 128, 129, 256, 700, 1], 2112, 2176),
    ([1057, 986, 1030, 1010], 2048, 2048),
    ([17, 5, 96], 2048, 2176)])
def test_gemm_wide_items_match_whole_tiles(L, counts, d, f):
    """An expert whose last rows fill at most half a 256-row tile runs them
    as wide items (those rows over two N panels, one per wave group). Every
    output element takes the same K order as in a whole tile, so the same
    rows give the same bits when the expert is padded (200 rows past its
    last whole tile) so that they fall in whole tiles instead: layer 0 (bf16
    SwiGLU output, rows gathered from x) and layer 1 (fp32 rows and compact
    rows), K of at least 2048 (wide items are used from there), with odd and
    partial panel counts (17 and 9 panels: a wide item with no second
    panel). With the workspace (every item split along K, the fixup pass
    finishing the wide items too) the results stay within fp32 summation
    error of the unsplit ones."""
    log(f"[edge] wide items counts={counts} d={d} f={f}")
    E = len(counts)
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(sum(counts) + d + f)
    bf = torch.bfloat16
    T = 3000
    x = torch.randn(T, d, generator=gen, device=dev).to(bf)
    Wg = (torch.randn(E, d, f, generator=gen, device=dev) * d ** -0.5).to(bf)
    Wu = (torch.randn(E, d, f, generator=gen, device=dev) * d ** -0.5).to(bf)
    Wd = (torch.randn(E, f, d, generator=gen, device=dev) * f ** -0.5).to(bf)
    pads = _wide_pads(counts)

    def layout(cnts):
        off = np.concatenate([[0], np.cumsum(cnts)]).astype(np.int32)
        return off, torch.tensor(off, dtype=torch.int32, device=dev)

    off1, off1_d = layout(counts)
    off2, off2_d = layout([c + p for c, p in zip(counts, pads)])
    R1, R2 = int(off1[-1]), int(off2[-1])
    # gather entries lie below min(T, rows), as moe_expert_up requires
    gather1 = torch.randint(0, min(T, R1), (R1,), generator=gen, device=dev, dtype=torch.int32)
    # the padded layout: each expert's rows first, then its pad rows
    where = np.concatenate([np.arange(off2[e], off2[e] + counts[e]) for e in range(E)]).astype(np.int64)
    where_d = torch.from_numpy(where).to(dev)
    gather2 = torch.randint(0, min(T, R2), (R2,), generator=gen, device=dev, dtype=torch.int32)
    gather2[where_d] = gather1

    def run(off_d, R, gather, ws, a_in=None):
        # layer 1 reads a_in when given (the same input for split and unsplit)
        wsb = L.moe_ffn_workspace_size(E, R, d, f) if ws else 0
        w = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        a = torch.empty(R, f, dtype=bf, device=dev)
        L.moe_expert_up(x, gather, off_d, E, R, d, f, L.MOE_BF16, Wg, Wu, a, w if ws else None, wsb)
        if a_in is not None:
            a = a_in
        yp = torch.empty(R, d, device=dev)
        L.moe_expert_down(a, off_d, E, R, f, d, L.MOE_BF16, Wd, yp, None, None, None,
                          w if ws else None, wsb)
        yh = torch.empty(R, d, dtype=torch.float16, device=dev)
        ys = torch.empty(R, d // 32, device=dev)
        L.moe_expert_down_f16(a, off_d, E, R, f, d, Wd, yh, ys, w if ws else None, wsb)
        torch.cuda.synchronize()
        return a, yp, yh, ys

    a1, y1, h1, s1 = run(off1_d, R1, gather1, False)
    a2, y2, h2, s2 = run(off2_d, R2, gather2, False)
    assert torch.equal(a1, a2[where_d])
    assert torch.equal(y1, y2[where_d])
    assert torch.equal(h1, h2[where_d]) and torch.equal(s1, s2[where_d])
    # with the workspace: the tail split (every item here) against the unsplit run
    a3, _, _, _ = run(off1_d, R1, gather1, True)
    _, y3, _, _ = run(off1_d, R1, gather1, True, a_in=a1)
    # another fp32 grouping of h and u: one bf16 ulp of a, plus fp32 summation
    # error (about 1e-5 of the scale) where SiLU(h) u lies near zero
    a_rms = float(a1.float().pow(2).mean().sqrt())
    excess = ((a3.float() - a1.float()).abs() - a1.float().abs() * 2.0 ** -7) / a_rms
    log(f"  split vs unsplit: a beyond one ulp by at most {float(excess.max()):.2e} of rms")
    assert float(excess.max()) <= 1e-4
    scale = float(y1.abs().max()) if R1 else 1.0
    assert float((y3 - y1).abs().max()) <= 1e-5 * scale
    # and against the definition, fp64 on the same bf16 operands
    for e in range(E):
        r0, r1 = int(off1[e]), int(off1[e + 1])
        if r0 == r1:
            continue
        z = x[gather1[r0:r1].long()].double()
        h = z @ Wg[e].double()
        u = z @ Wu[e].double()
        a_ref = h * torch.sigmoid(h) * u
        err = float((a1[r0:r1].double() - a_ref).abs().max() / a_ref.abs().max())
        assert err <= 2e-2, (e, err)
        y_ref = a1[r0:r1].double() @ Wd[e].double()
        err = float((y1[r0:r1].double() - y_ref).abs().max() / y_ref.abs().max())
        assert err <= 1e-4, (e, err)
