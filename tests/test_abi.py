"""The C-ABI library loads, exports every symbol include/moe.h declares, and
rejects bad arguments on the host with the documented status codes, before
anything is launched (so these run without a GPU).  Fake device addresses
are safe here because a rejected call never dereferences them."""
import os
import re

import pytest

from mixture_experts_layer_top_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

A = 0x7F0000000000  # 16-byte aligned fake address
MIS = A + 4         # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*]+\s+\*?(moe_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libmoe.so is not built (python -m mixture_experts_layer_top_amd.build)")
    return L.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    assert set(names) == set(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for st in range(5):
        assert L.status_string(st)
    assert "unknown" in L.status_string(99)


def route(**kw):
    args = dict(x=A, W_r=A, bias=None, T=16, d=64, E=8, k=2, score=0, dtype=1, topk_idx=A,
                topk_w=A, logits_out=None)
    args.update(kw)
    return L.moe_route(**args, stream=0, check=False)


def test_route_validation(lib):
    assert route(k=9) == L.MOE_ERR_INVALID            # k > E
    assert route(k=0) == L.MOE_ERR_INVALID
    assert route(E=0) == L.MOE_ERR_INVALID
    assert route(E=257, k=2) == L.MOE_ERR_INVALID
    assert route(T=-1) == L.MOE_ERR_INVALID
    assert route(x=None) == L.MOE_ERR_INVALID
    assert route(topk_w=None) == L.MOE_ERR_INVALID
    assert route(d=60) == L.MOE_ERR_UNSUPPORTED       # not a multiple of 8
    assert route(x=MIS) == L.MOE_ERR_UNSUPPORTED
    assert route(dtype=7) == L.MOE_ERR_UNSUPPORTED
    assert route(score=5) == L.MOE_ERR_UNSUPPORTED
    assert route(T=0) == L.MOE_OK                     # no-op, nothing launched
    assert route(T=1 << 30, k=4) == L.MOE_ERR_INVALID  # T*k overflows int32 rows


def permute(**kw):
    args = dict(topk_idx=A, topk_w=A, x=None, T=64, d=64, E=8, k=2, dtype=1, counts=A,
                offsets=A, perm_token=A, inv=A, perm_w=A, x_perm=None, workspace=A,
                ws_bytes=1 << 20)
    args.update(kw)
    return L.moe_permute(**args, stream=0, check=False)


def test_permute_validation(lib):
    need = L.moe_permute_workspace_size(64, 8, 2)
    assert need > 0
    assert permute(ws_bytes=need - 1) == L.MOE_ERR_WORKSPACE
    assert permute(workspace=None) == L.MOE_ERR_WORKSPACE
    assert permute(k=9) == L.MOE_ERR_INVALID
    assert permute(counts=None) == L.MOE_ERR_INVALID
    assert permute(inv=None) == L.MOE_ERR_INVALID
    assert permute(topk_w=None) == L.MOE_ERR_INVALID   # perm_w requested without weights
    assert permute(x_perm=A) == L.MOE_ERR_INVALID      # gather requested without x
    assert permute(x_perm=A, x=A, d=12) == L.MOE_ERR_UNSUPPORTED
    assert permute(perm_token=MIS) == L.MOE_ERR_UNSUPPORTED


def up(**kw):
    args = dict(x=A, gather_idx=None, offsets=A, E=8, rows=128, d=64, f=128, dtype=1, W_gate=A,
                W_up=A, a_out=A, workspace=A, ws_bytes=1 << 20)
    args.update(kw)
    return L.moe_expert_up(**args, stream=0, check=False)


def down(**kw):
    args = dict(a=A, offsets=A, E=8, rows=128, f=128, d=64, dtype=1, W_down=A, y_perm=A,
                scatter_idx=None, row_w=None, y=None, workspace=A, ws_bytes=1 << 20)
    args.update(kw)
    return L.moe_expert_down(**args, stream=0, check=False)


def test_ffn_validation(lib):
    assert up(W_up=None) == L.MOE_ERR_INVALID
    assert up(offsets=None) == L.MOE_ERR_INVALID
    assert up(f=100) == L.MOE_ERR_UNSUPPORTED
    assert up(d=-8) == L.MOE_ERR_INVALID
    assert up(E=0) == L.MOE_ERR_INVALID
    assert up(a_out=MIS) == L.MOE_ERR_UNSUPPORTED
    assert up(rows=0) == L.MOE_OK
    assert down(y_perm=None, y=None) == L.MOE_ERR_INVALID  # no output requested
    assert down(y=MIS, y_perm=None) == L.MOE_ERR_UNSUPPORTED
    assert down(dtype=3) == L.MOE_ERR_UNSUPPORTED
    assert down(rows=0) == L.MOE_OK
    st = L.moe_ffn_forward(A, None, A, 8, 128, 64, 128, 1, A, A, None, A, A, None, None, None, A,
                           1 << 20, stream=0, check=False)
    assert st == L.MOE_ERR_INVALID  # W_down missing


def test_combine_validation(lib):
    c = lambda **kw: L.moe_combine(**dict(dict(y_perm=A, inv=A, topk_w=A, T=16, d=64, k=2,  # noqa
                                               y_shared=None, shared_gate_logit=None,
                                               accumulate=0, y=A), **kw), stream=0, check=False)
    assert c(y=None) == L.MOE_ERR_INVALID
    assert c(topk_w=None) == L.MOE_ERR_INVALID
    assert c(shared_gate_logit=A) == L.MOE_ERR_INVALID  # gate without a shared term
    assert c(accumulate=2) == L.MOE_ERR_INVALID
    assert c(d=20) == L.MOE_ERR_UNSUPPORTED
    assert c(T=0) == L.MOE_OK


def test_compact_rows_validation(lib):
    dn = lambda **kw: L.moe_expert_down_f16(**dict(dict(  # noqa
        a=A, offsets=A, E=8, rows=128, f=128, d=64, W_down=A, y_h=A, y_s=A, workspace=A,
        ws_bytes=1 << 20), **kw), stream=0, check=False)
    assert dn(y_h=None) == L.MOE_ERR_INVALID
    assert dn(y_s=None) == L.MOE_ERR_INVALID
    assert dn(W_down=None) == L.MOE_ERR_INVALID
    assert dn(offsets=None) == L.MOE_ERR_INVALID
    assert dn(E=0) == L.MOE_ERR_INVALID
    assert dn(d=72) == L.MOE_ERR_UNSUPPORTED   # not whole 32-column segments
    assert dn(f=100) == L.MOE_ERR_UNSUPPORTED  # bf16 rows of 16-byte vectors
    assert dn(y_s=MIS) == L.MOE_ERR_UNSUPPORTED
    assert dn(y_h=MIS) == L.MOE_ERR_UNSUPPORTED
    assert dn(rows=0) == L.MOE_OK
    assert dn(rows=0, d=72) == L.MOE_ERR_UNSUPPORTED
    c = lambda **kw: L.moe_combine_f16(**dict(dict(  # noqa
        y_h=A, y_s=A, inv=A, topk_w=A, T=16, d=64, k=2, ys_h=None, ys_s=None,
        shared_gate_logit=None, accumulate=0, y=A), **kw), stream=0, check=False)
    assert c(y=None) == L.MOE_ERR_INVALID
    assert c(y_s=None) == L.MOE_ERR_INVALID
    assert c(topk_w=None) == L.MOE_ERR_INVALID
    assert c(ys_h=A) == L.MOE_ERR_INVALID               # shared rows without their factors
    assert c(ys_s=A) == L.MOE_ERR_INVALID
    assert c(shared_gate_logit=A) == L.MOE_ERR_INVALID  # gate without a shared term
    assert c(accumulate=2) == L.MOE_ERR_INVALID
    assert c(k=0) == L.MOE_ERR_INVALID
    assert c(d=72) == L.MOE_ERR_UNSUPPORTED
    assert c(ys_h=A, ys_s=MIS) == L.MOE_ERR_UNSUPPORTED
    assert c(T=0) == L.MOE_OK


def test_backward_validation(lib):
    """The training entry points reject bad arguments on the host."""
    cb = dict(dy=A, y_perm=A, inv=A, topk_w=A, T=16, d=64, k=2, dtype=L.MOE_BF16, y_shared=None,
              shared_gate_logit=None, dy_perm=A, dw=A, dy_shared=None, dgate_logit=None)
    def combine_bwd(**kw):
        return L.moe_combine_backward(**{**cb, **kw}, stream=0, check=False)
    assert combine_bwd(k=257) == L.MOE_ERR_INVALID
    assert combine_bwd(k=9, T=0) == L.MOE_OK  # any k up to 256
    assert combine_bwd(k=0) == L.MOE_ERR_INVALID
    assert combine_bwd(dy=None) == L.MOE_ERR_INVALID
    assert combine_bwd(d=60) == L.MOE_ERR_UNSUPPORTED
    assert combine_bwd(dw=MIS) == L.MOE_ERR_UNSUPPORTED
    assert combine_bwd(shared_gate_logit=A) == L.MOE_ERR_INVALID  # gate without its outputs
    assert combine_bwd(dtype=7) == L.MOE_ERR_UNSUPPORTED
    assert combine_bwd(T=0) == L.MOE_OK
    ch = dict(dy=A, y_h=A, y_s=A, inv=A, topk_w=A, T=16, d=64, k=2, dtype=L.MOE_BF16,
              ys_h=None, ys_s=None, shared_gate_logit=None, dy_perm=A, dw=A, dy_shared=None,
              dgate_logit=None)
    def combine_bwd16(**kw):
        return L.moe_combine_backward_f16(**{**ch, **kw}, stream=0, check=False)
    assert combine_bwd16(k=257) == L.MOE_ERR_INVALID
    assert combine_bwd16(k=20, T=0) == L.MOE_OK
    assert combine_bwd16(k=0) == L.MOE_ERR_INVALID
    assert combine_bwd16(y_h=None) == L.MOE_ERR_INVALID
    assert combine_bwd16(y_s=None) == L.MOE_ERR_INVALID
    assert combine_bwd16(ys_h=A) == L.MOE_ERR_INVALID        # shared rows without factors
    assert combine_bwd16(shared_gate_logit=A, dy_shared=A, dgate_logit=A) == L.MOE_ERR_INVALID
    assert combine_bwd16(dgate_logit=A) == L.MOE_ERR_INVALID  # gradient without a gate
    assert combine_bwd16(d=72) == L.MOE_ERR_UNSUPPORTED       # not whole 32-column segments
    assert combine_bwd16(y_s=MIS) == L.MOE_ERR_UNSUPPORTED
    assert combine_bwd16(dtype=7) == L.MOE_ERR_UNSUPPORTED
    assert combine_bwd16(T=0, d=72) == L.MOE_OK
    db = dict(dy_perm=A, offsets=A, E=8, rows=32, f=64, d=64, dtype=L.MOE_BF16, W_down=A, h=A,
              u=A, act=A, dhu=A, dW_down=A, workspace=None, ws_bytes=0)
    def down_bwd(**kw):
        return L.moe_expert_down_backward(**{**db, **kw}, stream=0, check=False)
    assert down_bwd(dtype=5) == L.MOE_ERR_UNSUPPORTED
    assert down_bwd(f=60) == L.MOE_ERR_UNSUPPORTED
    assert down_bwd(E=0) == L.MOE_ERR_INVALID
    assert down_bwd(offsets=None) == L.MOE_ERR_INVALID
    assert down_bwd(h=None) == L.MOE_ERR_INVALID
    assert down_bwd(dhu=MIS) == L.MOE_ERR_UNSUPPORTED
    assert down_bwd(workspace=MIS, ws_bytes=1 << 20) == L.MOE_ERR_UNSUPPORTED
    ub = dict(x=A, gather_idx=None, offsets=A, E=8, rows=32, d=64, f=64, dtype=L.MOE_BF16,
              W_gate=A, W_up=A, dhu=A, dx_perm=A, accumulate=0, dW_gate=A, dW_up=A,
              workspace=None, ws_bytes=0)
    def up_bwd(**kw):
        return L.moe_expert_up_backward(**{**ub, **kw}, stream=0, check=False)
    assert up_bwd(accumulate=2) == L.MOE_ERR_INVALID
    assert up_bwd(dW_up=None) == L.MOE_ERR_INVALID
    assert up_bwd(x=MIS) == L.MOE_ERR_UNSUPPORTED
    assert up_bwd(d=12) == L.MOE_ERR_UNSUPPORTED
    unp = dict(dx_perm=A, inv=A, T=16, d=64, k=2, accumulate=0, dx=A)
    def unpermute(**kw):
        return L.moe_unpermute(**{**unp, **kw}, stream=0, check=False)
    assert unpermute(k=257) == L.MOE_ERR_INVALID
    assert unpermute(k=9, T=0) == L.MOE_OK
    assert unpermute(inv=None) == L.MOE_ERR_INVALID
    assert unpermute(d=20) == L.MOE_ERR_UNSUPPORTED
    assert unpermute(T=0) == L.MOE_OK
    tk = dict(logits=A, topk_idx=A, dw=A, T=16, E=8, k=2, score=0, dL=A)
    def topk_bwd(**kw):
        return L.moe_topk_weights_backward(**{**tk, **kw}, stream=0, check=False)
    assert topk_bwd(k=9) == L.MOE_ERR_INVALID
    assert topk_bwd(score=5) == L.MOE_ERR_UNSUPPORTED
    assert topk_bwd(dL=None) == L.MOE_ERR_INVALID
    lb = dict(x=A, W=A, G=A, T=16, d=64, E=8, dtype=L.MOE_BF16, dW=A, db=None, dx=A,
              workspace=A, ws_bytes=1 << 24)
    def lin_bwd(**kw):
        return L.moe_linear_backward(**{**lb, **kw}, stream=0, check=False)
    assert lin_bwd(E=257) == L.MOE_ERR_INVALID
    assert lin_bwd(G=None) == L.MOE_ERR_INVALID
    assert lin_bwd(d=12) == L.MOE_ERR_UNSUPPORTED        # rows move as 16-byte vectors
    assert lin_bwd(x=MIS) == L.MOE_ERR_UNSUPPORTED
    assert lin_bwd(dx=MIS) == L.MOE_ERR_UNSUPPORTED
    assert lin_bwd(ws_bytes=16) == L.MOE_ERR_WORKSPACE
    # bf16 splits G into the workspace even without dW
    assert lin_bwd(dW=None, workspace=None, ws_bytes=0) == L.MOE_ERR_WORKSPACE
    assert lin_bwd(workspace=MIS) == L.MOE_ERR_UNSUPPORTED
    assert lin_bwd(T=0) == L.MOE_OK
    assert L.moe_linear_backward_workspace_size(16, 64, 8) > 0


def test_binding_raises_on_error(lib):
    with pytest.raises(L.MoeError):
        L.moe_route(A, A, None, 16, 64, 8, 9, 0, 1, A, A, None, stream=0)


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "mixture_experts_layer_top_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in src and "from oracle" not in src, fn
                assert "moe_oracle" not in src, fn


@pytest.mark.parametrize("T,d,f,E,k,dt", [
    (4096, 4096, 14336, 8, 2, 1), (8192, 3584, 2560, 64, 8, 1), (32768, 2048, 1408, 64, 6, 1),
    (100000, 64, 48, 256, 8, 1), (128, 64, 128, 4, 2, 0), (1, 8, 8, 1, 1, 1)])
def test_one_workspace_serves_every_forward_call(lib, T, d, f, E, k, dt):
    ws = L.moe_workspace_size(T, d, f, E, k, dt)
    assert ws % 16 == 0
    assert ws >= L.moe_permute_workspace_size(T, E, k)
    assert ws >= L.moe_ffn_workspace_size(E, T * k, d, f)
    # the FFN part is shape independent: the same buffer serves a shared-expert FFN
    assert ws >= L.moe_ffn_workspace_size(1, T, d, 20480)


def test_workspace_size_edge_cases(lib):
    assert L.moe_workspace_size(0, 4096, 14336, 8, 2, 1) == 0    # T = 0: every call is a no-op
    assert L.moe_workspace_size(-1, 64, 64, 8, 2, 1) == 0        # rejected arguments
    assert L.moe_workspace_size(16, 64, 64, 8, 9, 1) == 0        # k > E
    assert L.moe_workspace_size(16, 64, 64, 257, 2, 1) == 0      # E > 256
    assert L.moe_workspace_size(16, 64, 64, 8, 2, 7) == 0        # unknown dtype
    # with T = 0 (rows = 0) the calls that read a workspace return before any
    # launch and accept none (moe_permute still clears counts and offsets,
    # so it is not called here on fake addresses)
    assert up(rows=0, workspace=None, ws_bytes=0) == L.MOE_OK
    assert route(T=0) == L.MOE_OK


def test_probe_validation(lib):
    assert L.moe_probe_mfma(0, 10, None, A, stream=0, check=False) == L.MOE_ERR_INVALID
    assert L.moe_probe_mfma(4, 0, A, A, stream=0, check=False) == L.MOE_ERR_INVALID
    assert L.moe_probe_mfma(4, 10, A, None, stream=0, check=False) == L.MOE_ERR_INVALID
    assert L.moe_probe_mfma(4, 10, None, MIS, stream=0, check=False) == L.MOE_ERR_UNSUPPORTED
    assert L.moe_probe_mfma(4, 10, MIS, A, stream=0, check=False) == L.MOE_ERR_UNSUPPORTED
    # the streaming-read probe: validation before any launch (bytes = 0 is a no-op)
    assert L.moe_probe_read(A, 0, A, stream=0, check=False) == L.MOE_OK
    assert L.moe_probe_read(None, 64, A, stream=0, check=False) == L.MOE_ERR_INVALID
    assert L.moe_probe_read(A, 64, None, stream=0, check=False) == L.MOE_ERR_INVALID
    assert L.moe_probe_read(A, 60, A, stream=0, check=False) == L.MOE_ERR_UNSUPPORTED
    assert L.moe_probe_read(MIS, 64, A, stream=0, check=False) == L.MOE_ERR_UNSUPPORTED
    assert L.moe_probe_read(A, 64, MIS, stream=0, check=False) == L.MOE_ERR_UNSUPPORTED


def permute_noalloc(**kw):
    args = dict(topk_idx=A, topk_w=A, x=None, T=64, d=64, E=8, k=2, dtype=1, counts=A,
                offsets=A, perm_token=A, inv=A, perm_w=A, x_perm=None)
    args.update(kw)
    return L.moe_permute_noalloc(**args, stream=0, check=False)


def test_permute_noalloc_validation(lib):
    # the static scratch holds 1 MiB: 2 * ceil(T / 256) * E int32 tables
    assert permute_noalloc(T=131073, E=256, k=8) == L.MOE_ERR_WORKSPACE
    assert L.moe_permute_workspace_size(131072, 256, 8) <= 1 << 20
    assert L.moe_permute_workspace_size(131073, 256, 8) > 1 << 20
    assert permute_noalloc(k=9) == L.MOE_ERR_INVALID
    assert permute_noalloc(counts=None) == L.MOE_ERR_INVALID
    assert permute_noalloc(topk_w=None) == L.MOE_ERR_INVALID
    assert permute_noalloc(x_perm=A) == L.MOE_ERR_INVALID
    assert permute_noalloc(x_perm=A, x=A, d=12) == L.MOE_ERR_UNSUPPORTED
    assert permute_noalloc(perm_token=MIS) == L.MOE_ERR_UNSUPPORTED
    assert permute_noalloc(dtype=5) == L.MOE_ERR_UNSUPPORTED
