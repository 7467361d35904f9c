"""fp64 CPU oracle of the MoE expert-layer backward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; it shares no code, header, table or helper with the HIP
library.  It is the plain definition the GPU backward kernels are checked
against.

What it computes.  The pages are about training MoE models: COMET overlaps
the expert layer's communication and computation in training (COMET page,
"What Is COMET"), and DisagMoE runs a dedicated backward stream beside the
forward one (DisagMoE page, "2.2 AF-Pipe").  They give no formula for the
gradients; these are the exact gradients of the forward the oracle module
``moe_oracle`` defines, for an upstream gradient dy of the output y: the
vector-Jacobian product of every input (x, the router W_r and bias b, the
expert weights, the shared-expert weights and gate vector) written out
step by step by the chain rule, in the forward's order reversed:

1. combine:   y[t] = sum_j w[t,j] Y[inv[t,j]]
              dw[t,j] = <dy[t], Y[inv[t,j]]>,  dY[inv[t,j]] = w[t,j] dy[t];
2. expert e, row r (token t = perm_token[r]):
              h = x_t W_gate[e], u = x_t W_up[e], a = SiLU(h) u, Y_r = a W_down[e]
              dW_down[e] += a^T dY_r,  da = dY_r W_down[e]^T,
              dh = da u SiLU'(h),  du = da SiLU(h),  SiLU'(h) = s (1 + h (1 - s)), s = sigmoid(h),
              dW_gate[e] += x_t^T dh,  dW_up[e] += x_t^T du,
              dx_t += dh W_gate[e]^T + du W_up[e]^T;
3. weights (the selection is piecewise constant: no gradient flows through
   it; the weights are smooth functions of the logits at a fixed selection):
              renormalised: w_j = softmax over the k selected logits,
                            dL_{e_j} = w_j (dw_j - sum_i w_i dw_i), other dL_e = 0;
              not renormalised: w_j = p_{e_j}, p = softmax(L) over all E,
                            dL_e = p_e ([e selected] dw_{j(e)} - sum_i p_{e_i} dw_i);
4. router:    dW_r = x^T dL,  db = sum_t dL[t],  dx += dL W_r^T;
5. shared experts (y += g * sum_s F_s(x), g = sigmoid(x . w_s) or 1):
              dS = g dy, each F_s as in step 2 on every token;
              gated: dz_t = <dy_t, S_t> g_t (1 - g_t), dw_s = x^T dz, dx += dz w_s.

Matmuls are library primitives used as steps; everything else is plain
numpy float64.
"""
from __future__ import annotations

import numpy as np

from . import moe_oracle as F


def dsilu(h: np.ndarray) -> np.ndarray:
    """d SiLU(h) / dh = s (1 + h (1 - s)), s = sigmoid(h)."""
    s = 1.0 / (1.0 + np.exp(-h))
    return s * (1.0 + h * (1.0 - s))


def swiglu_ffn_backward(z, Wg, Wu, Wd, dY):
    """For F(z) = (SiLU(z Wg) * (z Wu)) Wd and upstream dY (rows of z):
    returns dz, dWg, dWu, dWd (step 2 of the module docstring)."""
    z = np.asarray(z, np.float64)
    Wg = np.asarray(Wg, np.float64)
    Wu = np.asarray(Wu, np.float64)
    Wd = np.asarray(Wd, np.float64)
    h = z @ Wg
    u = z @ Wu
    a = F.silu(h) * u
    dWd = a.T @ dY
    da = dY @ Wd.T
    dh = da * u * dsilu(h)
    du = da * F.silu(h)
    dWg = z.T @ dh
    dWu = z.T @ du
    dz = dh @ Wg.T + du @ Wu.T
    return dz, dWg, dWu, dWd


def topk_weights_backward(L: np.ndarray, idx: np.ndarray, renorm: bool,
                          dw: np.ndarray) -> np.ndarray:
    """dL [T, E] for w = topk_weights(L, idx, renorm) and upstream dw [T, k]
    (step 3 of the module docstring)."""
    L = np.asarray(L, np.float64)
    T, E = L.shape
    m = L.max(axis=1, keepdims=True)
    ex = np.exp(L - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    dL = np.zeros((T, E), np.float64)
    rows = np.arange(T)[:, None]
    if renorm:
        ps = np.take_along_axis(p, idx, axis=1)
        w = ps / ps.sum(axis=1, keepdims=True)
        g = w * (dw - (w * dw).sum(axis=1, keepdims=True))
        dL[rows, idx] = g
    else:
        ps = np.take_along_axis(p, idx, axis=1)
        s = (ps * dw).sum(axis=1, keepdims=True)
        dL = -p * s
        dL[rows, idx] += ps * dw
    return dL


def backward(layer: dict, dy: np.ndarray, k: int, renorm: bool,
             idx: np.ndarray | None = None) -> dict:
    """Gradients of <dy, y> for the layer forward of ``moe_oracle.forward``.

    ``idx`` optionally fixes the selection (as in the forward).  Returns a
    dict with dx, dW_r, db (or None), dW_gate, dW_up, dW_down, and for
    shared experts dWs_gate, dWs_up [d, n_s*f_s], dWs_down [n_s, f_s, d],
    dw_s (or None); plus the intermediates dw [T, k], dY [R, d] (permuted
    rows), dL [T, E].
    """
    fw = F.forward(layer, k, renorm, idx=idx)
    x = np.asarray(layer["x"], np.float64)
    dy = np.asarray(dy, np.float64)
    W_r = np.asarray(layer["W_r"], np.float64)
    E = W_r.shape[1]
    T, d = x.shape
    L, idx, w = fw["L"], fw["idx"], fw["w"]
    inv, perm_token, perm_w, offsets, Y = fw["inv"], fw["perm_token"], fw["perm_w"], fw["offsets"], fw["Y"]

    # 1. combine
    dw = np.zeros((T, k), np.float64)
    for j in range(k):
        dw[:, j] = np.sum(dy * Y[inv[:, j]], axis=1)
    dY = perm_w[:, None] * dy[perm_token]

    # 2. experts, one permuted segment at a time
    dx = np.zeros((T, d), np.float64)
    dW_gate = np.zeros(layer["W_gate"].shape, np.float64)
    dW_up = np.zeros(layer["W_up"].shape, np.float64)
    dW_down = np.zeros(layer["W_down"].shape, np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = perm_token[lo:hi]
        dz, dWg, dWu, dWd = swiglu_ffn_backward(x[toks], layer["W_gate"][e], layer["W_up"][e],
                                                layer["W_down"][e], dY[lo:hi])
        dW_gate[e], dW_up[e], dW_down[e] = dWg, dWu, dWd
        np.add.at(dx, toks, dz)

    # 3. weights -> logits, 4. router
    dL = topk_weights_backward(L, idx, renorm, dw)
    dW_r = x.T @ dL
    db = dL.sum(axis=0) if layer.get("b") is not None else None
    dx += dL @ W_r.T

    out = dict(dx=dx, dW_r=dW_r, db=db, dW_gate=dW_gate, dW_up=dW_up, dW_down=dW_down,
               dw=dw, dY=dY, dL=dL)

    # 5. shared experts
    if layer.get("Ws_gate") is not None:
        Wsg = np.asarray(layer["Ws_gate"], np.float64)
        Wsu = np.asarray(layer["Ws_up"], np.float64)
        Wsd = np.asarray(layer["Ws_down"], np.float64)
        n_s, f_s, _ = Wsd.shape
        gated = layer.get("w_s") is not None
        if gated:
            w_s = np.asarray(layer["w_s"], np.float64)
            g = F.sigmoid(x @ w_s)
            S = F.shared_output(x, Wsg, Wsu, Wsd, None)
            dS = g[:, None] * dy
            dz = np.sum(dy * S, axis=1) * g * (1.0 - g)
            out["dw_s"] = x.T @ dz
            dx += dz[:, None] * w_s[None, :]
        else:
            dS = dy
            out["dw_s"] = None
        dWs_gate = np.zeros_like(Wsg)
        dWs_up = np.zeros_like(Wsu)
        dWs_down = np.zeros_like(Wsd)
        for s in range(n_s):
            cols = slice(s * f_s, (s + 1) * f_s)
            dz_s, dWg, dWu, dWd = swiglu_ffn_backward(x, Wsg[:, cols], Wsu[:, cols], Wsd[s], dS)
            dWs_gate[:, cols], dWs_up[:, cols], dWs_down[s] = dWg, dWu, dWd
            dx += dz_s
        out.update(dWs_gate=dWs_gate, dWs_up=dWs_up, dWs_down=dWs_down)
    out["dx"] = dx
    return out


# --------------------------------------------------------------------------
# selected gradient entries of a full-size layer, one by one
# --------------------------------------------------------------------------


def sampled_backward(layer: dict, dy: np.ndarray, k: int, renorm: bool, idx: np.ndarray,
                     tokens, expert_cols=(), expert_rows=(), shared_cols=(), shared_rows=()):
    """The same gradients as ``backward``, but only the entries asked for,
    each computed from its own definition so that full-size layers stay
    within reach of the CPU:

    * per token t of ``tokens``: dx[t] (routed, router and shared parts),
      dw[t], dL[t] and, for a gated shared expert, dz[t] = d<dy, y>/d(x_t . w_s);
    * per (e, j) of ``expert_cols``: column j of dW_gate[e] and of dW_up[e]
      (sums over expert e's rows of x^T dh[:, j], x^T du[:, j]);
    * per (e, i) of ``expert_rows``: row i of dW_down[e] (a[:, i]^T dY);
    * per column j of ``shared_cols`` / row i of ``shared_rows``: the same
      for the side-by-side shared experts (every token is a row).

    ``layer["W_gate"][e]`` etc. may be any per-expert accessor returning a
    [d, f] / [f, d] array (one expert converted at a time); ``idx`` fixes
    the selection (the weights are recomputed from the fp64 logits at it).
    The formulas are those of the module docstring, steps 1-5.
    """
    x = layer["x"]
    W_r = np.asarray(layer["W_r"], np.float64)
    b = layer.get("b")
    E = W_r.shape[1]
    T, d = x.shape
    tokens = np.asarray(tokens, np.int64)
    nt = len(tokens)
    f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731

    def weights_of(rows_t):
        L = f64(x[rows_t]) @ W_r + (0.0 if b is None else f64(b))
        return L, F.topk_weights(L, idx[rows_t], renorm)

    out = {}
    # -- tokens: routed experts, one expert's weights at a time
    Lt, wt = weights_of(tokens)
    xt = f64(x[tokens])
    dyt = f64(dy[tokens])
    dx = np.zeros((nt, d), np.float64)
    dw = np.zeros((nt, k), np.float64)
    for e in np.unique(idx[tokens]):
        Wg, Wu, Wd = f64(layer["W_gate"][e]), f64(layer["W_up"][e]), f64(layer["W_down"][e])
        for a_, j in zip(*np.nonzero(idx[tokens] == e)):
            h = xt[a_] @ Wg
            u = xt[a_] @ Wu
            Y = (F.silu(h) * u) @ Wd
            dw[a_, j] = dyt[a_] @ Y
            da = (wt[a_, j] * dyt[a_]) @ Wd.T
            dh = da * u * dsilu(h)
            du = da * F.silu(h)
            dx[a_] += Wg @ dh + Wu @ du
    dL = topk_weights_backward(Lt, idx[tokens], renorm, dw)
    dx += dL @ W_r.T
    out.update(dw=dw, dL=dL)
    # -- tokens: shared experts
    shared = layer.get("Ws_gate") is not None
    if shared:
        Wsg, Wsu = f64(layer["Ws_gate"]), f64(layer["Ws_up"])
        n_s, f_s, _ = layer["Ws_down"].shape
        gated = layer.get("w_s") is not None
        S = np.zeros((nt, d), np.float64)
        parts = []
        for s in range(n_s):
            cols = slice(s * f_s, (s + 1) * f_s)
            Wsd = f64(layer["Ws_down"][s])
            h = xt @ Wsg[:, cols]
            u = xt @ Wsu[:, cols]
            S += (F.silu(h) * u) @ Wsd
            parts.append((cols, Wsd, h, u))
        if gated:
            w_s = f64(layer["w_s"])
            g = F.sigmoid(xt @ w_s)
            dS = g[:, None] * dyt
            dz = np.sum(dyt * S, axis=1) * g * (1.0 - g)
            dx += dz[:, None] * w_s[None, :]
            out["dz"] = dz
        else:
            dS = dyt
        for cols, Wsd, h, u in parts:
            da = dS @ Wsd.T
            dx += (da * u * dsilu(h)) @ Wsg[:, cols].T + (da * F.silu(h)) @ Wsu[:, cols].T
    out["dx"] = dx

    # -- expert weight gradients: the expert's rows, then the asked columns / rows
    want = sorted({e for e, _ in expert_cols} | {e for e, _ in expert_rows})
    cols_out, rows_out = {}, {}
    for e in want:
        toks, slots = np.nonzero(idx == e)
        if len(toks) == 0:
            for (e2, j) in expert_cols:
                if e2 == e:
                    cols_out[(e, j)] = (np.zeros(d), np.zeros(d))
            for (e2, i) in expert_rows:
                if e2 == e:
                    rows_out[(e, i)] = np.zeros(d)
            continue
        _, w_rows = weights_of(toks)
        Xe = f64(x[toks])
        dYe = w_rows[np.arange(len(toks)), slots][:, None] * f64(dy[toks])
        Wg, Wu, Wd = layer["W_gate"][e], layer["W_up"][e], layer["W_down"][e]
        for (e2, j) in expert_cols:
            if e2 != e:
                continue
            h = Xe @ f64(Wg[:, j])
            u = Xe @ f64(Wu[:, j])
            da = dYe @ f64(Wd[j, :])
            cols_out[(e, j)] = (Xe.T @ (da * u * dsilu(h)), Xe.T @ (da * F.silu(h)))
        for (e2, i) in expert_rows:
            if e2 != e:
                continue
            a = F.silu(Xe @ f64(Wg[:, i])) * (Xe @ f64(Wu[:, i]))
            rows_out[(e, i)] = a @ dYe
    out.update(expert_cols=cols_out, expert_rows=rows_out)

    # -- shared weight gradients: every token is a row
    if shared and (shared_cols or shared_rows):
        X = f64(x)
        DY = f64(dy)
        if layer.get("w_s") is not None:
            DY = F.sigmoid(X @ f64(layer["w_s"]))[:, None] * DY
        Wsg, Wsu = f64(layer["Ws_gate"]), f64(layer["Ws_up"])
        n_s, f_s, _ = layer["Ws_down"].shape
        scol, srow = {}, {}
        for j in shared_cols:
            s, jj = divmod(j, f_s)
            h = X @ Wsg[:, j]
            u = X @ Wsu[:, j]
            da = DY @ f64(layer["Ws_down"][s][jj, :])
            scol[j] = (X.T @ (da * u * dsilu(h)), X.T @ (da * F.silu(h)))
        for i in shared_rows:
            a = F.silu(X @ Wsg[:, i]) * (X @ Wsu[:, i])
            srow[i] = a @ DY
        out.update(shared_cols=scol, shared_rows=srow)
    return out
