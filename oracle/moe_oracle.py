"""fp64 CPU oracle of the MoE expert-layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it exists so that the tests, the smoke check and the
benchmark's CPU-baseline leg can check (and time) the HIP kernels against a
plain, slow, obviously correct definition.  It shares no code, header,
table or helper with the HIP library.

What the layer computes, and where the pages say it:

* An MoE layer activates, per token, a sparse subset of its experts
  (DisagMoE page, "1. Declaração do Problema").
* The subset is the top-k experts of the router (DisagMoE page,
  "2.2 AF-Pipe", where k is named as the number of top-k experts); tokens are
  dispatched to those experts and the expert outputs are combined back
  (same passage, on dispatch and combine).
* The experts are FFN layers (DisagMoE page, "2.1 Posicionamento de
  Componentes Desagregados"), whose two GEMMs are "layer 0" and "layer 1"
  over a token dimension M and a hidden dimension N (COMET page,
  "COMET's Technical Principles", tensor decomposition).

The pages give no formula for the router score, the expert activation or
the shared experts.  This oracle takes these readings (each is listed with
its reason in the design notes):

* logits L = x W_r (+ b); selection = the first k experts under the order
  (descending L, ascending expert index) -- ties go to the lower index;
  selecting on logits equals selecting on softmax probabilities because
  softmax is strictly increasing;
* weights: p = softmax(L) over all E experts; w = p[sel] / sum(p[sel])
  (renormalised) or w = p[sel];
* expert e: SwiGLU, F_e(z) = (SiLU(z W_gate[e]) * (z W_up[e])) W_down[e],
  SiLU(h) = h / (1 + exp(-h)); no biases;
* dispatch: stable counting sort of the (token, slot) pairs by expert,
  tokens ascending inside each expert's segment (no capacity limit, no
  dropped tokens);
* combine: y[t] = sum_j w[t, j] * Y[inv[t, j]];
* shared experts: y[t] += g_t * sum_s F_s(x[t]), with g_t = sigmoid(x[t] . w_s)
  for the gated variant and g_t = 1 otherwise.

Every step is a plain numpy float64 expression or loop; matmul and sort are
library primitives used as steps.  Inputs are the exact tensors given to the
GPU, upcast to float64.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# routing: logits, top-k selection, weights
# --------------------------------------------------------------------------


def router_logits(x: np.ndarray, W_r: np.ndarray, b: np.ndarray | None = None) -> np.ndarray:
    """L[t, e] = sum_i x[t, i] W_r[i, e] + b[e], float64 (top-k router input,
    DisagMoE page, "2.2 AF-Pipe")."""
    L = np.asarray(x, np.float64) @ np.asarray(W_r, np.float64)
    if b is not None:
        L = L + np.asarray(b, np.float64)[None, :]
    return L


def select_topk(L: np.ndarray, k: int) -> np.ndarray:
    """idx[t, 0..k-1]: the first k experts of row t sorted by (-L[t, e], e).

    Row t holds its picks in rank order (largest logit first); exactly equal
    logits go to the lower expert index.
    """
    L = np.asarray(L, np.float64)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    e_idx = np.broadcast_to(np.arange(E), L.shape)
    # lexsort: last key is primary -> primary -L (descending L), secondary e
    order = np.lexsort((e_idx, -L), axis=1)
    return order[:, :k].astype(np.int64)


def topk_weights(L: np.ndarray, idx: np.ndarray, renorm: bool) -> np.ndarray:
    """Softmax over all E logits, gathered at the selection; renormalised over
    the k picks when ``renorm``.  Max-subtracted for range safety (exact in
    real arithmetic)."""
    L = np.asarray(L, np.float64)
    m = L.max(axis=1, keepdims=True)
    ex = np.exp(L - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, idx, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


# --------------------------------------------------------------------------
# dispatch: histogram, prefix scan, stable permutation
# --------------------------------------------------------------------------


def expert_counts(idx: np.ndarray, E: int) -> np.ndarray:
    """c_e = number of (t, j) pairs with idx[t, j] == e."""
    counts = np.zeros(E, np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero(idx == e))
    return counts


def exclusive_offsets(counts: np.ndarray) -> np.ndarray:
    """off[0] = 0, off[e + 1] = off[e] + c_e."""
    off = np.zeros(len(counts) + 1, np.int64)
    for e in range(len(counts)):
        off[e + 1] = off[e] + counts[e]
    return off


def permutation(idx: np.ndarray, E: int):
    """Stable counting sort of the (t, j) pairs by expert.

    Walks experts in order, and for each expert the tokens in ascending
    order; the pair (t, j) with idx[t, j] == e gets the next row r.
    Returns perm_token[R] (row -> token), inv[T, k] ((t, j) -> row) and the
    per-row slot perm_slot[R] (row -> j).
    """
    T, k = idx.shape
    R = T * k
    perm_token = np.full(R, -1, np.int64)
    perm_slot = np.full(R, -1, np.int64)
    inv = np.full((T, k), -1, np.int64)
    r = 0
    for e in range(E):
        ts, js = np.nonzero(idx == e)  # row-major: ascending t
        n = len(ts)
        perm_token[r:r + n] = ts
        perm_slot[r:r + n] = js
        inv[ts, js] = np.arange(r, r + n)
        r += n
    assert r == R, "every (token, slot) pair must name an expert in [0, E)"
    return perm_token, inv, perm_slot


# --------------------------------------------------------------------------
# expert FFN (SwiGLU) and combine
# --------------------------------------------------------------------------


def silu(h: np.ndarray) -> np.ndarray:
    """SiLU(h) = h / (1 + exp(-h))."""
    return h / (1.0 + np.exp(-h))


def swiglu_ffn(z: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
               chunk: int = 4096) -> np.ndarray:
    """F(z) = (SiLU(z Wg) * (z Wu)) Wd for every row of z, float64.

    The two products are the expert's "layer 0" and "layer 1" (COMET page,
    "COMET's Technical Principles").  Rows are processed in chunks only to
    bound memory; each row is independent.
    """
    Wg = np.asarray(Wg, np.float64)
    Wu = np.asarray(Wu, np.float64)
    Wd = np.asarray(Wd, np.float64)
    out = np.empty((z.shape[0], Wd.shape[1]), np.float64)
    for s in range(0, z.shape[0], chunk):
        zc = np.asarray(z[s:s + chunk], np.float64)
        h = zc @ Wg
        u = zc @ Wu
        out[s:s + chunk] = (silu(h) * u) @ Wd
    return out


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def combine(Y: np.ndarray, inv: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[t] = sum_j w[t, j] * Y[inv[t, j]] (the combine of DisagMoE page,
    "2.2 AF-Pipe")."""
    T, k = inv.shape
    y = np.zeros((T, Y.shape[1]), np.float64)
    for j in range(k):
        y += w[:, j:j + 1] * Y[inv[:, j]]
    return y


def shared_output(x, Ws_gate, Ws_up, Ws_down, w_s=None) -> np.ndarray:
    """sum_s F_s(x), scaled per token by sigmoid(x . w_s) when w_s is given.
    Ws_down is [n_s, f_s, d]; shared expert s's gate/up projections are
    columns s*f_s .. (s+1)*f_s - 1 of Ws_gate/Ws_up [d, n_s*f_s]."""
    x = np.asarray(x, np.float64)
    n_s, f_s, d = Ws_down.shape
    ys = np.zeros((x.shape[0], d), np.float64)
    for s in range(n_s):
        cols = slice(s * f_s, (s + 1) * f_s)
        ys += swiglu_ffn(x, Ws_gate[:, cols], Ws_up[:, cols], Ws_down[s])
    if w_s is not None:
        g = sigmoid(x @ np.asarray(w_s, np.float64))
        ys = g[:, None] * ys
    return ys


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------


def route(layer: dict, k: int, renorm: bool):
    """Logits, selection and weights for every token."""
    L = router_logits(layer["x"], layer["W_r"], layer.get("b"))
    idx = select_topk(L, k)
    w = topk_weights(L, idx, renorm)
    return L, idx, w


def dispatch(idx: np.ndarray, w: np.ndarray, E: int):
    """Counts, offsets and the stable permutation, plus per-row weights."""
    counts = expert_counts(idx, E)
    offsets = exclusive_offsets(counts)
    perm_token, inv, perm_slot = permutation(idx, E)
    perm_w = w[perm_token, perm_slot]
    return counts, offsets, perm_token, inv, perm_w


def expert_outputs(layer: dict, perm_token, offsets, E: int) -> np.ndarray:
    """Y[r] = F_e(x[perm_token[r]]) for every permuted row r of expert e."""
    x = layer["x"]
    d = layer["W_down"].shape[2]
    Y = np.zeros((len(perm_token), d), np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            Y[lo:hi] = swiglu_ffn(x[perm_token[lo:hi]], layer["W_gate"][e],
                                  layer["W_up"][e], layer["W_down"][e])
    return Y


def forward(layer: dict, k: int, renorm: bool, idx: np.ndarray | None = None):
    """The full layer forward in float64.

    ``layer`` holds float64 arrays (see ``to_f64`` of the input generator).
    ``idx`` optionally fixes the selection (used where several selections
    are correct, i.e. near-ties between fp32 and fp64 logits); weights are
    then taken at that selection from the fp64 logits.
    Returns a dict with L, idx, w, counts, offsets, perm_token, inv, perm_w, Y, y.
    """
    E = layer["W_r"].shape[1]
    L = router_logits(layer["x"], layer["W_r"], layer.get("b"))
    if idx is None:
        idx = select_topk(L, k)
    w = topk_weights(L, idx, renorm)
    counts, offsets, perm_token, inv, perm_w = dispatch(idx, w, E)
    Y = expert_outputs(layer, perm_token, offsets, E)
    y = combine(Y, inv, w)
    if layer.get("Ws_gate") is not None:
        y = y + shared_output(layer["x"], layer["Ws_gate"], layer["Ws_up"],
                              layer["Ws_down"], layer.get("w_s"))
    return dict(L=L, idx=idx, w=w, counts=counts, offsets=offsets, perm_token=perm_token,
                inv=inv, perm_w=perm_w, Y=Y, y=y)


def token_output(layer: dict, t: int, sel, w_t) -> np.ndarray:
    """y[t] for one token given its selection and weights (routed + shared);
    the per-token form used to check sampled rows of full-size layers."""
    xt = np.asarray(layer["x"][t:t + 1], np.float64)
    yt = np.zeros((1, layer["W_down"].shape[2]), np.float64)
    for e, we in zip(sel, w_t):
        yt += we * swiglu_ffn(xt, layer["W_gate"][e], layer["W_up"][e], layer["W_down"][e])
    if layer.get("Ws_gate") is not None:
        yt += shared_output(xt, layer["Ws_gate"], layer["Ws_up"], layer["Ws_down"],
                            layer.get("w_s"))
    return yt[0]


# --------------------------------------------------------------------------
# dense brute force (tiny inputs only)
# --------------------------------------------------------------------------


def brute_force(layer: dict, k: int, renorm: bool) -> dict:
    """Every expert on every token, masked by the top-k weights.

    Bypasses the histogram, scan, permutation and combine entirely and
    re-derives the selection with a per-token Python sort and the weights
    with scipy's softmax, so it shares no step of ``forward`` beyond the
    logits' definition.
    """
    from scipy.special import softmax

    x = np.asarray(layer["x"], np.float64)
    W_r = np.asarray(layer["W_r"], np.float64)
    L = x @ W_r
    if layer.get("b") is not None:
        L = L + np.asarray(layer["b"], np.float64)
    T, E = L.shape
    sel = np.array([sorted(range(E), key=lambda e: (-L[t, e], e))[:k] for t in range(T)],
                   dtype=np.int64).reshape(T, k)
    P = softmax(L, axis=1)
    G = np.zeros((T, E))
    for t in range(T):
        ps = P[t, sel[t]]
        if renorm:
            ps = ps / ps.sum()
        G[t, sel[t]] = ps
    d = layer["W_down"].shape[2]
    y = np.zeros((T, d))
    for e in range(E):
        h = x @ layer["W_gate"][e]
        u = x @ layer["W_up"][e]
        a = h * (1.0 / (1.0 + np.exp(-h))) * u
        y += G[:, e:e + 1] * (a @ layer["W_down"][e])
    if layer.get("Ws_gate") is not None:
        ys = np.zeros_like(y)
        n_s, f_s, _ = layer["Ws_down"].shape
        for s in range(n_s):
            h = x @ layer["Ws_gate"][:, s * f_s:(s + 1) * f_s]
            u = x @ layer["Ws_up"][:, s * f_s:(s + 1) * f_s]
            ys += (h * (1.0 / (1.0 + np.exp(-h))) * u) @ layer["Ws_down"][s]
        if layer.get("w_s") is not None:
            g = 1.0 / (1.0 + np.exp(-(x @ layer["w_s"])))
            ys = g[:, None] * ys
        y = y + ys
    return dict(L=L, idx=sel, G=G, y=y)


# --------------------------------------------------------------------------
# decision margins (for comparing fp32 GPU routing with fp64 routing)
# --------------------------------------------------------------------------


def selection_margin(L: np.ndarray, k: int) -> np.ndarray:
    """Smallest gap between adjacent values among the k+1 largest logits of
    each row (all E when k == E, since the rank order of the k picks is part
    of the selection; inf only for a single expert): a perturbation of every
    logit by less than half of it changes neither the selection nor its
    order, while moving the two logits at that gap by a little more than half
    of it swaps them."""
    T, E = L.shape
    s = -np.sort(-L, axis=1)
    top = s[:, :min(k + 1, E)]
    if top.shape[1] < 2:
        return np.full(T, np.inf)
    return np.min(top[:, :-1] - top[:, 1:], axis=1)


def fp32_logit_error_bound(x: np.ndarray, W_r: np.ndarray, b: np.ndarray | None = None,
                           safety: float = 2.0) -> np.ndarray:
    """Bound on |fl32(L[t, e]) - L[t, e]| per token, for a length-d dot product
    of exactly representable products summed in float32 in any order, plus the
    bias add: gamma_{d+1} * (sum_i |x_i| max_e |W_ie| + max_e |b_e|), with
    gamma_n = n u / (1 - n u) and u = 2^-24 (the classical forward error bound
    of recursive floating-point summation).  ``safety`` widens it for adders
    whose internal rounding is not plain round-to-nearest."""
    d = x.shape[1]
    u = 2.0 ** -24
    n = d + 1
    gamma = n * u / (1 - n * u)
    s = np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(W_r, np.float64)).max(axis=1)
    if b is not None:
        s = s + float(np.abs(np.asarray(b, np.float64)).max())
    return safety * gamma * s
