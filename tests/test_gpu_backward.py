"""Parity of the HIP backward pass (through the C ABI) with the fp64 CPU
backward oracle.

Every gradient the layer returns (x, router W_r and bias, expert gate/up/down
weights, shared experts and their gate vector) and the slot-weight gradient
dw are compared with the oracle evaluated at the GPU's selection, on seeded
upstream gradients dy.  Bars, per tensor (per expert for the experts'
weight gradients, whose scale differs between experts with many and few
tokens; an empty expert's gradients must be exactly zero):
  * normwise: ||g_gpu - g_ref||_F <= NORM_TAU * ||g_ref||_F, NORM_TAU = 1e-2;
  * elementwise: |g_gpu - g_ref| <= EL_TAU * (|g_ref| + rms(g_ref)),
    EL_TAU = 5e-2 (a gradient entry's error scales with the entry: a few
    tokens can dominate an expert's weight-gradient entry, so a bar against
    the rms alone would be set by the tensor's tails);
  * the router bias gradient db[e] = sum_t dL[t, e] is a sum with heavy
    cancellation, bounded against its terms' magnitudes:
    |db_gpu - db_ref| <= NORM_TAU * sum_t |dL_ref[t, e]|.
Where they come from: the forward's bar for bf16 storage is 2e-2 * rms for
one bf16 intermediate (the activation a); the backward chains three bf16
roundings (dy_perm = w dy, then dH and dU, with the saved h, u and a as
operands; 2^-9 relative each), with fp32 accumulation everywhere else.
Measured on the mid-size workloads: normwise 0.16-0.36%, elementwise
constant <= 3.4%, db <= 0.1%.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle.moe_backward as B
from mixture_experts_layer_top_amd.inputs import CONFIGS, make_layer

pytestmark = pytest.mark.gpu

NORM_TAU = 1e-2
EL_TAU = 5e-2

MID = {
    "mixtral": CONFIGS["mixtral"].shrink(T=2000, d=520, f=392),
    "qwen2moe": CONFIGS["qwen2moe"].shrink(T=1024, d=264, f=200, f_shared=256),
    "mixtral_skew": CONFIGS["mixtral_skew"].shrink(T=3000, d=256, f=256),
    "deepseek": CONFIGS["deepseek"].shrink(T=1500, d=256, f=136, f_shared=136),
    "mixtral_k64": CONFIGS["mixtral"].shrink(T=2000, d=512, f=320),
}

# oracle gradient key -> (GPU gradient key, reshape of the GPU tensor to the oracle's)
KEYS = {"dx": "dx", "dW_r": "dW_r", "db": "db", "dW_gate": "dW_gate", "dW_up": "dW_up",
        "dW_down": "dW_down", "dWs_gate": "dWs_gate", "dWs_up": "dWs_up",
        "dWs_down": "dWs_down", "dw_s": "dw_s"}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def L():
    from mixture_experts_layer_top_amd import _lib
    _lib.load()
    return _lib


def rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def host(layer):
    return {k: (None if v is None else v.to("cpu", torch.float64).numpy()) for k, v in layer.items()}


def run_train(cfg, layer, dy):
    from mixture_experts_layer_top_amd.layer import MoeLayer
    m = MoeLayer(cfg, layer, path="fast", train=True)
    m.forward()
    g = m.backward(dy)
    torch.cuda.synchronize()
    return m, g


def errors(got, ref):
    """normwise relative error, max error over rms, and the smallest c with
    |got - ref| <= c (|ref| + rms(ref)) everywhere"""
    diff = np.abs(got - ref)
    r = rms(ref)
    nrm = float(np.linalg.norm(diff) / np.linalg.norm(ref))
    mx = float(np.max(diff)) / r
    c = float(np.max(diff / (np.abs(ref) + r)))
    return nrm, mx, c


PER_EXPERT = ("dW_gate", "dW_up", "dW_down")


def check_grads(cfg, m, g, h, dy_h, norm_tau=NORM_TAU, el_tau=EL_TAU):
    """Log every statistic first, then assert the bars of the module
    docstring (per expert for the experts' weight gradients)."""
    idx = m.idx.cpu().numpy().astype(np.int64)
    ref = B.backward(h, dy_h, cfg.k, cfg.renorm, idx=idx)
    fails = []
    got_dw = m.dw.cpu().double().numpy()
    items = [("dw", got_dw, ref["dw"])]
    for rk, gk in KEYS.items():
        if ref.get(rk) is None:
            assert g.get(gk) is None, gk
            continue
        items.append((rk, g[gk].cpu().double().numpy().reshape(ref[rk].shape), ref[rk]))
    for rk, got, rf in items:
        if rk in PER_EXPERT:
            worst = [0.0, 0.0, 0.0]
            for e in range(cfg.E):
                if not np.any(rf[e]):
                    if np.any(got[e]):
                        fails.append(f"{rk}[{e}] must be exactly zero (empty expert)")
                    continue
                st = errors(got[e], rf[e])
                worst = [max(a, b) for a, b in zip(worst, st)]
                if st[0] > norm_tau or st[2] > el_tau:
                    fails.append(f"{rk}[{e}]: normwise {st[0]:.3e}, c {st[2]:.3e}")
            log(f"  {cfg.name} {rk} (worst expert): normwise {worst[0]:.3e}, max/rms {worst[1]:.3e}, "
                f"c {worst[2]:.3e}")
        elif rk == "db":
            scale = np.sum(np.abs(ref["dL"]), axis=0)
            ratio = float(np.max(np.abs(got - rf) / np.maximum(scale, 1e-300)))
            log(f"  {cfg.name} db: max |d| / sum_t |dL| = {ratio:.3e}")
            if ratio > norm_tau:
                fails.append(f"db: {ratio:.3e}")
        elif not np.any(rf):
            # e.g. one expert with renormalised weights: w = 1 exactly, so the
            # router gets no gradient at all
            log(f"  {cfg.name} {rk}: reference exactly zero, GPU max |g| {np.max(np.abs(got)):.3e}")
            if np.any(got):
                fails.append(f"{rk} must be exactly zero")
        else:
            st = errors(got, rf)
            log(f"  {cfg.name} {rk}: normwise {st[0]:.3e}, max/rms {st[1]:.3e}, c {st[2]:.3e}")
            if st[0] > norm_tau or st[2] > el_tau:
                fails.append(f"{rk}: normwise {st[0]:.3e}, c {st[2]:.3e}")
    assert not fails, fails


@pytest.mark.parametrize("name", list(MID))
def test_backward_parity_mid(L, name):
    cfg = MID[name]
    log(f"[bwd] {name} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
    layer = make_layer(cfg, seed=0, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(11)
    dy = torch.randn(cfg.T, cfg.d, generator=gen, device="cuda", dtype=torch.float32)
    m, g = run_train(cfg, layer, dy)
    check_grads(cfg, m, g, host(layer), dy.cpu().double().numpy())


# fp32 layers: fp32 storage and accumulation everywhere, so the bars are
# those of the fp32 forward (1e-4) instead of the bf16 chain's
F32_NORM_TAU = 1e-4
F32_EL_TAU = 1e-3
MID_F32 = {
    "tiny": CONFIGS["tiny"],
    "qwen2moe_f32": dataclasses.replace(CONFIGS["qwen2moe"].shrink(T=300, d=72, f=56, f_shared=40),
                                        dtype="f32"),
    "deepseek_f32": dataclasses.replace(CONFIGS["deepseek"].shrink(T=257, d=64, f=40, f_shared=24),
                                        dtype="f32"),
}


@pytest.mark.parametrize("name", list(MID_F32))
def test_backward_parity_f32(L, name):
    """The fp32 layer's training step (the tiny workload at its full size,
    and fp32 versions of the shared-expert shapes) against the oracle."""
    cfg = MID_F32[name]
    log(f"[bwd f32] {name} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
    layer = make_layer(cfg, seed=0, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(13)
    dy = torch.randn(cfg.T, cfg.d, generator=gen, device="cuda", dtype=torch.float32)
    m, g = run_train(cfg, layer, dy)
    check_grads(cfg, m, g, host(layer), dy.cpu().double().numpy(), F32_NORM_TAU, F32_EL_TAU)


def _edge_cfg(**kw):
    base = dict(name="edge", cfg_id=9, T=130, d=72, f=40, E=8, k=2, renorm=True, dtype="bf16")
    base.update(kw)
    return CONFIGS["mixtral"].__class__(**base)


def _edge_run(cfg, seed):
    layer = make_layer(cfg, seed=seed, device="cuda")
    dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator(device="cuda").manual_seed(seed),
                     device="cuda", dtype=torch.float32)
    m, g = run_train(cfg, layer, dy)
    check_grads(cfg, m, g, host(layer), dy.cpu().double().numpy())


@pytest.mark.parametrize("E,k,T", [(1, 1, 300), (4, 4, 300), (256, 8, 300), (3, 2, 300),
                                   (4, 2, 1), (8, 2, 63)])
def test_backward_expert_and_token_extremes(L, E, k, T):
    """One expert; k = E; 256 experts of about nine rows each; an odd E; a
    single token; a ragged T: the backward against the oracle."""
    log(f"[bwd edge] E={E} k={k} T={T}")
    _edge_run(_edge_cfg(E=E, k=k, T=T, d=64, f=48), seed=100 + E + T)


@pytest.mark.parametrize("E,k,shared", [(16, 10, False), (64, 20, True), (32, 32, False)])
def test_backward_more_than_eight_slots(L, E, k, shared):
    """k above 8: the combine backward and the unpermute take the slots one
    after another (k = 10, 20 and k = E = 32); with a gated shared expert,
    the shared gate's gradient through the same kernel."""
    log(f"[bwd edge] E={E} k={k} shared={shared}")
    kw = dict(E=E, k=k, T=200, d=64, f=48)
    if shared:
        kw.update(n_shared=1, f_shared=64, shared_gated=True)
    _edge_run(_edge_cfg(**kw), seed=300 + E + k)


@pytest.mark.parametrize("nk", [1, 2, 3, 5])
def test_backward_stage_counts(L, nk):
    """d = f = 64 nk: the scalar-base backward GEMMs with 1, 2, 3 and 5 K
    stages of the data gradients (their prologues take other branches for
    nk < 3) and weight-gradient K ranges of about 175 rows."""
    log(f"[bwd edge] stages nk={nk}")
    _edge_run(_edge_cfg(E=16, k=4, T=700, d=64 * nk, f=64 * nk), seed=200 + nk)


def test_backward_is_deterministic(L):
    cfg = MID["deepseek"]
    layer = make_layer(cfg, seed=2, device="cuda")
    dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator(device="cuda").manual_seed(3),
                     device="cuda", dtype=torch.float32)
    _, g1 = run_train(cfg, layer, dy)
    g1 = {k: (None if v is None else v.clone()) for k, v in g1.items()}
    _, g2 = run_train(cfg, layer, dy)
    for k, v in g1.items():
        if v is not None:
            assert torch.equal(v, g2[k]), k


def test_backward_zero_upstream(L):
    cfg = MID["qwen2moe"]
    layer = make_layer(cfg, seed=4, device="cuda")
    m, g = run_train(cfg, layer, torch.zeros(cfg.T, cfg.d, device="cuda"))
    for k, v in g.items():
        if v is not None:
            assert torch.count_nonzero(v).item() == 0, k


def test_backward_empty_expert_gets_zero_weight_gradients(L):
    """A skewed router at twice the stated bias leaves the last expert empty:
    its weight gradients are exactly zero, the others are not."""
    from mixture_experts_layer_top_amd.inputs import sweep_configs
    base = {c.bias_scale: c for c in sweep_configs("skew")}[2.0]
    cfg = base.shrink(T=512, d=128, f=128)
    layer = make_layer(cfg, seed=0, device="cuda")
    dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator(device="cuda").manual_seed(5),
                     device="cuda", dtype=torch.float32)
    m, g = run_train(cfg, layer, dy)
    counts = m.counts.cpu().numpy()
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) > 0, counts
    for e in range(cfg.E):
        for k in ("dW_gate", "dW_up", "dW_down"):
            nz = torch.count_nonzero(g[k][e]).item()
            assert (nz == 0) == (counts[e] == 0), (k, e, counts[e], nz)
    check_grads(cfg, m, g, host(layer), dy.cpu().double().numpy())


def test_expert_up_backward_gather_matches_permuted_copy(L):
    """moe_expert_up_backward reading x through the permutation (the
    128 x 128 kernel's row gather) and reading the permuted copy x_perm (the
    256 x 256 ping-pong kernel) give the same gradients: the data gradient
    bit for bit (the same kernel), the weight gradients to fp32 rounding
    (both sum each expert's rows in row order, 64 at a time)."""
    cfg = MID["mixtral"]
    layer = make_layer(cfg, seed=6, device="cuda")
    dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator(device="cuda").manual_seed(8),
                     device="cuda", dtype=torch.float32)
    m, g = run_train(cfg, layer, dy)
    R = cfg.T * cfg.k
    dx_perm = torch.empty_like(m.dx_perm)
    dWg = torch.empty_like(g["dW_gate"])
    dWu = torch.empty_like(g["dW_up"])
    L.moe_expert_up_backward(layer["x"], m.perm_token, m.offsets, cfg.E, R, cfg.d, cfg.f,
                             L.MOE_BF16, layer["W_gate"], layer["W_up"], m.dhu, dx_perm, 0, dWg,
                             dWu, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(dx_perm, m.dx_perm)
    for got, ref in ((dWg, g["dW_gate"]), (dWu, g["dW_up"])):
        err = (got - ref).abs().max().item() / ref.abs().max().item()
        log(f"  gather vs copy weight gradient: max rel {err:.3e}")
        assert err <= 1e-6


@pytest.mark.parametrize("counts", [[4173], [3100, 1073], [0, 4173]])
def test_weight_gradient_k_split(L, counts):
    """With the workspace, launches with few weight-gradient tiles cut each
    expert's rows into K chunks and add the fp32 partials in chunk order.
    The data gradients (dhu, dx_perm) are unchanged bit for bit; the weight
    gradients equal their fp64 definition on the same bf16 operands
    (dW_down[e] = act_e^T dy_e, dW_gate[e] = x_e^T dH_e, dW_up[e] = x_e^T dU_e)
    to fp32 summation error, split or not; an empty expert's are zero."""
    d, f = 512, 384
    E, rows = len(counts), sum(counts)
    ws_bytes = L.moe_ffn_backward_workspace_size(E, rows, d, f)
    assert ws_bytes > 0  # 4-6 tiles per expert: the split is taken
    gen = torch.Generator(device="cuda").manual_seed(rows + E)

    def rnd(*shape, scale=1.0):
        return (torch.randn(*shape, generator=gen, device="cuda") * scale).to(torch.bfloat16)

    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32,
                           device="cuda")
    dy, x = rnd(rows, d), rnd(rows, d)
    h, u, act = rnd(rows, f), rnd(rows, f), rnd(rows, f)
    W_down, W_gate, W_up = rnd(E, f, d, scale=f ** -0.5), rnd(E, d, f, scale=d ** -0.5), \
        rnd(E, d, f, scale=d ** -0.5)
    out = {}
    for split in (False, True):
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if split else None
        dhu = torch.empty(rows, 2 * f, dtype=torch.bfloat16, device="cuda")
        dWd = torch.full((E, f, d), float("nan"), device="cuda")
        dxp = torch.empty(rows, d, device="cuda")
        dWg = torch.full((E, d, f), float("nan"), device="cuda")
        dWu = torch.full((E, d, f), float("nan"), device="cuda")
        L.moe_expert_down_backward(dy, offsets, E, rows, f, d, L.MOE_BF16, W_down, h, u, act, dhu,
                                   dWd, ws, ws_bytes if split else 0)
        L.moe_expert_up_backward(x, None, offsets, E, rows, d, f, L.MOE_BF16, W_gate, W_up, dhu,
                                 dxp, 0, dWg, dWu, ws, ws_bytes if split else 0)
        torch.cuda.synchronize()
        out[split] = dict(dhu=dhu, dx=dxp, dW_down=dWd, dW_gate=dWg, dW_up=dWu)
    assert torch.equal(out[False]["dhu"], out[True]["dhu"])
    assert torch.equal(out[False]["dx"], out[True]["dx"])
    dhu = out[True]["dhu"].cpu().double()
    ops = {"dW_down": (act, dy), "dW_gate": (x, dhu[:, :f]), "dW_up": (x, dhu[:, f:])}
    off = offsets.cpu().tolist()
    for key, (a, b) in ops.items():
        a = a.cpu().double() if torch.is_tensor(a) and a.is_cuda else a
        b = b.cpu().double() if torch.is_tensor(b) and b.is_cuda else b
        for e in range(E):
            ref = (a[off[e]:off[e + 1]].T @ b[off[e]:off[e + 1]]).numpy()
            for split in (False, True):
                got = out[split][key][e].cpu().double().numpy()
                if counts[e] == 0:
                    assert np.count_nonzero(got) == 0, (key, e, split)
                    continue
                err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
                log(f"  {key}[{e}] split={split}: normwise {err:.2e}")
                assert err <= 1e-5, (key, e, split, err)


@pytest.mark.parametrize("E", [1, 3, 8, 16, 32, 100])
def test_linear_backward_any_expert_count(L, E):
    """moe_linear_backward (the router's linear map L = x W + b, backward):
    dW = x^T G, db = column sums of G, dx += G W^T, against the fp64
    definition on the same bf16 x, W and fp32 G; every expert-block width
    (8, 16, 32, 64, and 64 twice for E = 100) and a ragged T and d."""
    T, d = 777, 200
    gen = torch.Generator(device="cuda").manual_seed(E)
    x = torch.randn(T, d, generator=gen, device="cuda").to(torch.bfloat16)
    W = (torch.randn(d, E, generator=gen, device="cuda") / d ** 0.5).to(torch.bfloat16)
    G = torch.randn(T, E, generator=gen, device="cuda")
    dx0 = torch.randn(T, d, generator=gen, device="cuda")
    dW = torch.empty(d, E, device="cuda")
    db = torch.empty(E, device="cuda")
    dx = dx0.clone()
    ws_bytes = L.moe_linear_backward_workspace_size(T, d, E)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    L.moe_linear_backward(x, W, G, T, d, E, L.MOE_BF16, dW, db, dx, ws, ws_bytes)
    torch.cuda.synchronize()
    xh, Wh, Gh = (t.cpu().double().numpy() for t in (x, W, G))
    refs = {"dW": (dW, xh.T @ Gh), "db": (db, Gh.sum(0)),
            "dx": (dx, dx0.cpu().double().numpy() + Gh @ Wh.T)}
    for name, (got, ref) in refs.items():
        nrm, _, c = errors(got.cpu().double().numpy(), ref)
        log(f"  linear backward E={E} {name}: normwise {nrm:.2e}, c {c:.2e}")
        # fp32 sums of at most T products of bf16 x or W with G (G split
        # exactly into bf16 hi + lo, residual <= 2^-18 |G|): far inside 1e-5
        assert nrm <= 1e-5 and c <= 1e-4, (name, nrm, c)


# ---------------------------------------------------------------- full size


class _PerExpert:
    """fp64 view of a [E, a, b] device tensor, converted one expert at a time."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        return self.t[e].to("cpu", torch.float64).numpy()


def _host_lazy(layer):
    return {k_: (None if v is None else (_PerExpert(v) if v.dim() == 3 else
                                         v.to("cpu", torch.float64).numpy()))
            for k_, v in layer.items()}


def _bars(name, got, ref, fails):
    nrm, mx, c = errors(got, ref)
    log(f"  {name}: normwise {nrm:.3e}, max/rms {mx:.3e}, c {c:.3e}")
    if nrm > NORM_TAU or c > EL_TAU:
        fails.append(f"{name}: normwise {nrm:.3e}, c {c:.3e}")


@pytest.mark.parametrize("name", ["mixtral", "qwen2moe", "mixtral_skew", "deepseek"])
def test_backward_full_size_sampled(L, name):
    """The training step at full size, in the launch configuration the
    benchmark times, checked on entries the oracle computes one by one: dx,
    dw, dL and the shared gate's dz of sampled tokens; columns of dW_gate and
    dW_up and rows of dW_down of the most- and least-loaded experts and a
    random one; columns and rows of the shared experts' weight gradients.
    The whole-tensor reductions over every token (dW_r = x^T dL, db, dw_s =
    x^T dz) and the top-k weights backward on every token are checked
    against their fp64 definitions applied to the GPU's own dL, dz and dw
    (which the samples tie to the oracle)."""
    cfg = CONFIGS[name]
    log(f"[bwd full] {name} T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
    layer = make_layer(cfg, seed=0, device="cuda")
    dy = torch.randn(cfg.T, cfg.d, generator=torch.Generator(device="cuda").manual_seed(11),
                     device="cuda", dtype=torch.float32)
    m, g = run_train(cfg, layer, dy)
    h = _host_lazy(layer)
    dyh = dy.cpu().double().numpy()
    idx = m.idx.cpu().numpy().astype(np.int64)
    counts = m.counts.cpu().numpy()
    rng = np.random.default_rng(7)
    nonempty = np.nonzero(counts > 0)[0]
    e_big = int(np.argmax(counts))
    e_small = int(nonempty[np.argmin(counts[nonempty])])
    experts = sorted({e_big, e_small, int(rng.choice(nonempty))})
    toks = {0, cfg.T - 1} | set(rng.choice(cfg.T, 6, replace=False).tolist())
    toks |= set(np.nonzero(np.any(idx == e_small, axis=1))[0][:2].tolist())
    toks = np.array(sorted(toks))
    js = [0, cfg.f - 1, int(rng.integers(cfg.f))]
    ec = [(e, j) for e in experts for j in js]
    fs_all = cfg.n_shared * cfg.f_shared if cfg.n_shared else 0
    sj = [0, fs_all - 1, int(rng.integers(fs_all))] if fs_all else []
    ref = B.sampled_backward(h, dyh, cfg.k, cfg.renorm, idx, toks, ec, ec, sj, sj)
    log(f"  oracle done: {len(toks)} tokens, experts {experts} (counts {counts[experts].tolist()})")
    fails = []
    _bars("dx[sampled tokens]", g["dx"].cpu().double().numpy()[toks], ref["dx"], fails)
    dw_g = m.dw.cpu().double().numpy()
    _bars("dw[sampled tokens]", dw_g[toks], ref["dw"], fails)
    dL_g = m.dL.cpu().double().numpy()
    # dL = w (dw - <w, dw>) (or the full-softmax form): an error eps in dw
    # moves an entry by at most 2 eps max|dw| (w, p <= 1)
    lim = 2 * NORM_TAU * np.max(np.abs(ref["dw"]), axis=1)
    worst = float(np.max(np.max(np.abs(dL_g[toks] - ref["dL"]), axis=1) / lim))
    log(f"  dL[sampled tokens]: max |d| / (2 tau max|dw|) = {worst:.3e}")
    if worst > 1.0:
        fails.append(f"dL: {worst:.3e}")
    for e, j in ec:
        _bars(f"dW_gate[{e}][:, {j}]", g["dW_gate"][e][:, j].cpu().double().numpy(),
              ref["expert_cols"][(e, j)][0], fails)
        _bars(f"dW_up[{e}][:, {j}]", g["dW_up"][e][:, j].cpu().double().numpy(),
              ref["expert_cols"][(e, j)][1], fails)
        _bars(f"dW_down[{e}][{j}, :]", g["dW_down"][e][j, :].cpu().double().numpy(),
              ref["expert_rows"][(e, j)], fails)
    for j in sj:
        _bars(f"dWs_gate[:, {j}]", g["dWs_gate"][:, j].cpu().double().numpy(),
              ref["shared_cols"][j][0], fails)
        _bars(f"dWs_up[:, {j}]", g["dWs_up"][:, j].cpu().double().numpy(),
              ref["shared_cols"][j][1], fails)
        _bars(f"dWs_down[{j}, :]", g["dWs_down"][j, :].cpu().double().numpy(),
              ref["shared_rows"][j], fails)
    # reductions over every token, on the GPU's own inputs (exact operands)
    x = h["x"]
    L32 = m.logits.cpu().double().numpy()
    dL_def = B.topk_weights_backward(L32, idx, cfg.renorm, dw_g)
    scale = np.max(np.abs(dw_g), axis=1, keepdims=True) + 1e-30
    tk = float(np.max(np.abs(dL_g - dL_def) / scale))
    log(f"  top-k weights backward, every token: max |d| / max|dw| = {tk:.3e}")
    if tk > 1e-5:
        fails.append(f"top-k weights backward: {tk:.3e}")
    nrm, _, c = errors(g["dW_r"].cpu().double().numpy(), x.T @ dL_g)
    log(f"  dW_r vs x^T dL: normwise {nrm:.3e}, c {c:.3e}")
    if nrm > 1e-5 or c > 1e-4:
        fails.append(f"dW_r: {nrm:.3e} {c:.3e}")
    if g.get("db") is not None:
        r = float(np.max(np.abs(g["db"].cpu().double().numpy() - dL_g.sum(0)) /
                         (np.abs(dL_g).sum(0) + 1e-30)))
        log(f"  db vs sum_t dL: {r:.3e}")
        if r > 1e-5:
            fails.append(f"db: {r:.3e}")
    if "dz" in ref:
        dz_g = m.dgl.cpu().double().numpy().reshape(-1)
        _bars("dz[sampled tokens]", dz_g[toks], ref["dz"], fails)
        nrm, _, c = errors(g["dw_s"].cpu().double().numpy().reshape(-1), x.T @ dz_g)
        log(f"  dw_s vs x^T dz: normwise {nrm:.3e}, c {c:.3e}")
        if nrm > 1e-5 or c > 1e-4:
            fails.append(f"dw_s: {nrm:.3e} {c:.3e}")
    assert not fails, fails


@pytest.mark.parametrize("T,d,k,shared,dt", [
    (77, 96, 1, "none", "bf16"), (77, 96, 2, "gated", "bf16"), (130, 2048, 6, "plain", "bf16"),
    (130, 4128, 8, "gated", "bf16"), (50, 512, 10, "gated", "bf16"), (33, 160, 20, "plain", "f32"),
    (64, 64, 8, "gated", "f32")])
def test_combine_backward_compact_rows(L, T, d, k, shared, dt):
    """moe_combine_backward_f16 against moe_combine_backward over the
    restored rows (y_h * factor): dy_perm and dy_shared are the same products
    w dy and g dy, bit for bit; dw and the gate gradient are dot products of
    the same exact values in another summation order, so both lie within fp32
    summation error of their fp64 definition.  k of 1..8 (one pass) and
    above 8 (slot by slot); d of one thread's chunk, of exactly one chunk per
    thread (2048) and of a ragged second pass (4128)."""
    log(f"[bwd compact] T={T} d={d} k={k} shared={shared} {dt}")
    gen = torch.Generator(device="cuda").manual_seed(T * 31 + d + k)
    R, S = T * k, d // 32
    dtype = L.MOE_BF16 if dt == "bf16" else L.MOE_F32
    act = torch.bfloat16 if dt == "bf16" else torch.float32
    dy = torch.randn(T, d, generator=gen, device="cuda")
    # compact rows: fp16 values and power-of-two factors 2^-20 .. 2^-6
    y_h = (torch.rand(R, d, generator=gen, device="cuda") * 6e4 - 3e4).to(torch.float16)
    y_s = torch.exp2(torch.randint(-20, -5, (R, S), generator=gen, device="cuda").float())
    y_perm = y_h.float() * y_s.repeat_interleave(32, dim=1)
    inv = torch.randperm(R, generator=gen, device="cuda").to(torch.int32).reshape(T, k)
    w = torch.rand(T, k, generator=gen, device="cuda")
    ys_h = ys_s = ys = gl = None
    if shared == "gated":
        ys_h = (torch.rand(T, d, generator=gen, device="cuda") * 6e4 - 3e4).to(torch.float16)
        ys_s = torch.exp2(torch.randint(-20, -5, (T, S), generator=gen, device="cuda").float())
        ys = ys_h.float() * ys_s.repeat_interleave(32, dim=1)
        gl = torch.randn(T, 1, generator=gen, device="cuda")
    out = {}
    for name in ("f16", "f32"):
        o = dict(dy_perm=torch.full((R, d), float("nan"), device="cuda").to(act),
                 dw=torch.full((T, k), float("nan"), device="cuda"),
                 dys=torch.full((T, d), float("nan"), device="cuda").to(act)
                 if shared != "none" else None,
                 dgl=torch.full((T, 1), float("nan"), device="cuda") if gl is not None else None)
        if name == "f16":
            L.moe_combine_backward_f16(dy, y_h, y_s, inv, w, T, d, k, dtype, ys_h, ys_s, gl,
                                       o["dy_perm"], o["dw"], o["dys"], o["dgl"])
        else:
            L.moe_combine_backward(dy, y_perm, inv, w, T, d, k, dtype, ys, gl, o["dy_perm"],
                                   o["dw"], o["dys"], o["dgl"])
        torch.cuda.synchronize()
        out[name] = o
    assert torch.equal(out["f16"]["dy_perm"], out["f32"]["dy_perm"])
    if shared != "none":
        assert torch.equal(out["f16"]["dys"], out["f32"]["dys"])
    # fp64 definitions and their fp32 summation bound: d 2^-24 sum |terms|
    dyh, yph, invh = dy.cpu().double(), y_perm.cpu().double(), inv.cpu().long()
    rows = yph[invh]                                    # [T, k, d]
    ref = (rows * dyh[:, None, :]).sum(-1)
    bound = 2 * d * 2.0 ** -24 * (rows * dyh[:, None, :]).abs().sum(-1) + 1e-30
    for name in ("f16", "f32"):
        err = float(((out[name]["dw"].cpu().double() - ref).abs() / bound).max())
        log(f"  dw {name}: max err / bound {err:.3f}")
        assert err <= 1.0, (name, err)
    if gl is not None:
        g = torch.sigmoid(gl.cpu().double())[:, 0]
        prod = ys.cpu().double() * dyh
        ref_g = prod.sum(-1) * g * (1 - g)
        bound_g = (2 * d * 2.0 ** -24 * prod.abs().sum(-1) + 2e-5 * prod.sum(-1).abs()) \
            * g * (1 - g) + 1e-30
        for name in ("f16", "f32"):
            err = float(((out[name]["dgl"].cpu().double()[:, 0] - ref_g).abs() / bound_g).max())
            log(f"  dgate {name}: max err / bound {err:.3f}")
            assert err <= 1.0, (name, err)
