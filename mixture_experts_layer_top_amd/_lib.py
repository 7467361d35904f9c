"""ctypes binding of libmoe.so.

Argument marshalling only: each function has the name and argument order of
the C entry point (include/moe.h), accepts torch tensors (or None for NULL)
and ints, passes device pointers and the current HIP stream, and raises
``MoeError`` on a non-zero status.  No step of the layer runs here.  A
missing library is an error: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX_TOPK_RENORM, MOE_SOFTMAX_TOPK = 0, 1

# every symbol include/moe.h declares
EXPORTS = (
    "moe_status_string", "moe_route", "moe_permute_workspace_size",
    "moe_permute",
    "moe_ffn_workspace_size", "moe_expert_up", "moe_expert_down", "moe_ffn_forward",
    "moe_combine", "moe_expert_up_save",
    "moe_combine_backward", "moe_expert_down_backward", "moe_expert_up_backward",
    "moe_unpermute", "moe_topk_weights_backward", "moe_linear_backward_workspace_size",
    "moe_linear_backward", "moe_ffn_backward_workspace_size", "moe_workspace_size",
    "moe_probe_mfma", "moe_permute_noalloc", "moe_probe_read",
    "moe_expert_down_f16", "moe_combine_f16", "moe_combine_backward_f16",
)

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def load():
    """Load libmoe.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mixture_experts_layer_top_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_route": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]),
        "moe_permute_workspace_size": (sz, [i32, i32, i32]),
        "moe_permute": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                              sz, vp]),
        "moe_ffn_workspace_size": (sz, [i32, i32, i32, i32]),
        "moe_workspace_size": (sz, [i32, i32, i32, i32, i32, i32]),
        "moe_probe_mfma": (i32, [i32, i32, vp, vp, vp]),
        "moe_probe_read": (i32, [vp, sz, vp, vp]),
        "moe_permute_noalloc": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                      vp]),
        "moe_expert_up": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
        "moe_expert_down": (i32, [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz,
                                  vp]),
        "moe_ffn_forward": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                  vp, vp, vp, sz, vp]),
        "moe_combine": (i32, [vp, vp, vp, i32, i32, i32, vp, vp, i32, vp, vp]),
        "moe_expert_down_f16": (i32, [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
        "moe_combine_f16": (i32, [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, i32, vp, vp]),
        "moe_expert_up_save": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                     vp, sz, vp]),
        "moe_combine_backward": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                       vp, vp]),
        "moe_combine_backward_f16": (i32, [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp,
                                           vp, vp, vp, vp, vp]),
        "moe_expert_down_backward": (i32, [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                           vp, vp, sz, vp]),
        "moe_expert_up_backward": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                         i32, vp, vp, vp, sz, vp]),
        "moe_ffn_backward_workspace_size": (sz, [i32, i32, i32, i32]),
        "moe_unpermute": (i32, [vp, vp, i32, i32, i32, i32, vp, vp]),
        "moe_topk_weights_backward": (i32, [vp, vp, vp, i32, i32, i32, i32, vp, vp]),
        "moe_linear_backward_workspace_size": (sz, [i32, i32, i32]),
        "moe_linear_backward": (i32, [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(t):
    """Device (or host) address of a tensor, an int address, or NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st, status_string(st))


def status_string(st: int) -> str:
    return load().moe_status_string(st).decode()


moe_status_string = status_string


def moe_route(x, W_r, bias, T, d, E, k, score, dtype, topk_idx, topk_w, logits_out,
              stream=None, check=True):
    st = load().moe_route(_p(x), _p(W_r), _p(bias), T, d, E, k, score, dtype, _p(topk_idx),
                          _p(topk_w), _p(logits_out), _stream(stream))
    if check:
        _check("moe_route", st)
    return st


def moe_permute_workspace_size(T, E, k):
    return load().moe_permute_workspace_size(T, E, k)


def moe_permute(topk_idx, topk_w, x, T, d, E, k, dtype, counts, offsets, perm_token, inv,
                perm_w, x_perm, workspace, ws_bytes, stream=None, check=True):
    st = load().moe_permute(_p(topk_idx), _p(topk_w), _p(x), T, d, E, k, dtype, _p(counts),
                            _p(offsets), _p(perm_token), _p(inv), _p(perm_w), _p(x_perm),
                            _p(workspace), ws_bytes, _stream(stream))
    if check:
        _check("moe_permute", st)
    return st


def moe_permute_noalloc(topk_idx, topk_w, x, T, d, E, k, dtype, counts, offsets, perm_token, inv,
                        perm_w, x_perm, stream=None, check=True):
    st = load().moe_permute_noalloc(_p(topk_idx), _p(topk_w), _p(x), T, d, E, k, dtype, _p(counts),
                                    _p(offsets), _p(perm_token), _p(inv), _p(perm_w), _p(x_perm),
                                    _stream(stream))
    if check:
        _check("moe_permute_noalloc", st)
    return st


def moe_ffn_workspace_size(E, rows, d, f):
    return load().moe_ffn_workspace_size(E, rows, d, f)


def moe_workspace_size(T, d, f, E, k, dtype):
    return load().moe_workspace_size(T, d, f, E, k, dtype)


def moe_expert_up(x, gather_idx, offsets, E, rows, d, f, dtype, W_gate, W_up, a_out, workspace,
                  ws_bytes, stream=None, check=True):
    st = load().moe_expert_up(_p(x), _p(gather_idx), _p(offsets), E, rows, d, f, dtype,
                              _p(W_gate), _p(W_up), _p(a_out), _p(workspace), ws_bytes,
                              _stream(stream))
    if check:
        _check("moe_expert_up", st)
    return st


def moe_expert_down(a, offsets, E, rows, f, d, dtype, W_down, y_perm, scatter_idx, row_w, y,
                    workspace, ws_bytes, stream=None, check=True):
    st = load().moe_expert_down(_p(a), _p(offsets), E, rows, f, d, dtype, _p(W_down), _p(y_perm),
                                _p(scatter_idx), _p(row_w), _p(y), _p(workspace), ws_bytes,
                                _stream(stream))
    if check:
        _check("moe_expert_down", st)
    return st


def moe_ffn_forward(x, gather_idx, offsets, E, rows, d, f, dtype, W_gate, W_up, W_down, a_buf,
                    y_perm, scatter_idx, row_w, y, workspace, ws_bytes, stream=None, check=True):
    st = load().moe_ffn_forward(_p(x), _p(gather_idx), _p(offsets), E, rows, d, f, dtype,
                                _p(W_gate), _p(W_up), _p(W_down), _p(a_buf), _p(y_perm),
                                _p(scatter_idx), _p(row_w), _p(y), _p(workspace), ws_bytes,
                                _stream(stream))
    if check:
        _check("moe_ffn_forward", st)
    return st


def moe_combine(y_perm, inv, topk_w, T, d, k, y_shared, shared_gate_logit, accumulate, y,
                stream=None, check=True):
    st = load().moe_combine(_p(y_perm), _p(inv), _p(topk_w), T, d, k, _p(y_shared),
                            _p(shared_gate_logit), accumulate, _p(y), _stream(stream))
    if check:
        _check("moe_combine", st)
    return st


def moe_expert_down_f16(a, offsets, E, rows, f, d, W_down, y_h, y_s, workspace, ws_bytes,
                        stream=None, check=True):
    st = load().moe_expert_down_f16(_p(a), _p(offsets), E, rows, f, d, _p(W_down), _p(y_h),
                                    _p(y_s), _p(workspace), ws_bytes, _stream(stream))
    if check:
        _check("moe_expert_down_f16", st)
    return st


def moe_combine_f16(y_h, y_s, inv, topk_w, T, d, k, ys_h, ys_s, shared_gate_logit, accumulate, y,
                    stream=None, check=True):
    st = load().moe_combine_f16(_p(y_h), _p(y_s), _p(inv), _p(topk_w), T, d, k, _p(ys_h),
                                _p(ys_s), _p(shared_gate_logit), accumulate, _p(y),
                                _stream(stream))
    if check:
        _check("moe_combine_f16", st)
    return st


# ---------------------------------------------------------------- training


def moe_expert_up_save(x, gather_idx, offsets, E, rows, d, f, dtype, W_gate, W_up, a_out, h_out,
                       u_out, workspace, ws_bytes, stream=None, check=True):
    st = load().moe_expert_up_save(_p(x), _p(gather_idx), _p(offsets), E, rows, d, f, dtype,
                                   _p(W_gate), _p(W_up), _p(a_out), _p(h_out), _p(u_out),
                                   _p(workspace), ws_bytes, _stream(stream))
    if check:
        _check("moe_expert_up_save", st)
    return st


def moe_combine_backward(dy, y_perm, inv, topk_w, T, d, k, dtype, y_shared, shared_gate_logit,
                         dy_perm, dw, dy_shared, dgate_logit, stream=None, check=True):
    st = load().moe_combine_backward(_p(dy), _p(y_perm), _p(inv), _p(topk_w), T, d, k, dtype,
                                     _p(y_shared), _p(shared_gate_logit), _p(dy_perm), _p(dw),
                                     _p(dy_shared), _p(dgate_logit), _stream(stream))
    if check:
        _check("moe_combine_backward", st)
    return st


def moe_combine_backward_f16(dy, y_h, y_s, inv, topk_w, T, d, k, dtype, ys_h, ys_s,
                             shared_gate_logit, dy_perm, dw, dy_shared, dgate_logit, stream=None,
                             check=True):
    st = load().moe_combine_backward_f16(_p(dy), _p(y_h), _p(y_s), _p(inv), _p(topk_w), T, d, k,
                                         dtype, _p(ys_h), _p(ys_s), _p(shared_gate_logit),
                                         _p(dy_perm), _p(dw), _p(dy_shared), _p(dgate_logit),
                                         _stream(stream))
    if check:
        _check("moe_combine_backward_f16", st)
    return st


def moe_ffn_backward_workspace_size(E, rows, d, f):
    return load().moe_ffn_backward_workspace_size(E, rows, d, f)


def moe_expert_down_backward(dy_perm, offsets, E, rows, f, d, dtype, W_down, h, u, act, dhu,
                             dW_down, workspace=None, ws_bytes=0, stream=None, check=True):
    st = load().moe_expert_down_backward(_p(dy_perm), _p(offsets), E, rows, f, d, dtype,
                                         _p(W_down), _p(h), _p(u), _p(act), _p(dhu), _p(dW_down),
                                         _p(workspace), ws_bytes, _stream(stream))
    if check:
        _check("moe_expert_down_backward", st)
    return st


def moe_expert_up_backward(x, gather_idx, offsets, E, rows, d, f, dtype, W_gate, W_up, dhu,
                           dx_perm, accumulate, dW_gate, dW_up, workspace=None, ws_bytes=0,
                           stream=None, check=True):
    st = load().moe_expert_up_backward(_p(x), _p(gather_idx), _p(offsets), E, rows, d, f, dtype,
                                       _p(W_gate), _p(W_up), _p(dhu), _p(dx_perm), accumulate,
                                       _p(dW_gate), _p(dW_up), _p(workspace), ws_bytes,
                                       _stream(stream))
    if check:
        _check("moe_expert_up_backward", st)
    return st


def moe_unpermute(dx_perm, inv, T, d, k, accumulate, dx, stream=None, check=True):
    st = load().moe_unpermute(_p(dx_perm), _p(inv), T, d, k, accumulate, _p(dx), _stream(stream))
    if check:
        _check("moe_unpermute", st)
    return st


def moe_topk_weights_backward(logits, topk_idx, dw, T, E, k, score, dL, stream=None, check=True):
    st = load().moe_topk_weights_backward(_p(logits), _p(topk_idx), _p(dw), T, E, k, score,
                                          _p(dL), _stream(stream))
    if check:
        _check("moe_topk_weights_backward", st)
    return st


def moe_linear_backward_workspace_size(T, d, E):
    return load().moe_linear_backward_workspace_size(T, d, E)


def moe_linear_backward(x, W, G, T, d, E, dtype, dW, db, dx, workspace, ws_bytes, stream=None,
                        check=True):
    st = load().moe_linear_backward(_p(x), _p(W), _p(G), T, d, E, dtype, _p(dW), _p(db), _p(dx),
                                    _p(workspace), ws_bytes, _stream(stream))
    if check:
        _check("moe_linear_backward", st)
    return st


# ---------------------------------------------------------------- measurement


def moe_probe_mfma(blocks, iters, operands, ticks, stream=None, check=True):
    st = load().moe_probe_mfma(blocks, iters, _p(operands), _p(ticks), _stream(stream))
    if check:
        _check("moe_probe_mfma", st)
    return st


def moe_probe_read(src, nbytes, sink, stream=None, check=True):
    st = load().moe_probe_read(_p(src), nbytes, _p(sink), _stream(stream))
    if check:
        _check("moe_probe_read", st)
    return st
