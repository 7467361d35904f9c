"""The measurement probes on the GPU: they run to completion at ragged and
large sizes and write nothing but their documented outputs."""
import pytest
import torch

from mixture_experts_layer_top_amd import _lib

pytestmark = pytest.mark.gpu


def test_probe_read_sizes():
    src = torch.ones(((1 << 26) + 64) // 4, dtype=torch.int32, device="cuda:0")  # 64 MiB + 64 B
    sink = torch.full((4,), -7, dtype=torch.int32, device="cuda:0")
    for nbytes in (16, 48, 4096 + 16, 1 << 20, (1 << 26) + 64):
        print(f"[probe_read] {nbytes} bytes", flush=True)
        _lib.moe_probe_read(src, nbytes, sink)
        torch.cuda.synchronize()
        # a buffer of ones folds to 0 or 1 per word, never the sink's trigger value
        assert sink.tolist() == [-7, -7, -7, -7]


@pytest.mark.parametrize("with_operands", [False, True])
def test_probe_mfma_ticks(with_operands):
    print(f"[probe_mfma] operands={with_operands}", flush=True)
    blocks = 8
    ops = None
    if with_operands:
        g = torch.Generator(device="cuda:0").manual_seed(0)
        ops = torch.randn(blocks * 16 * 256 * 8, generator=g, device="cuda:0").to(torch.bfloat16)
    ticks = torch.full((3 * blocks,), -1, dtype=torch.int64, device="cuda:0")
    _lib.moe_probe_mfma(blocks, 50, ops, ticks)
    torch.cuda.synchronize()
    t = ticks.view(blocks, 3).cpu()
    assert bool((t[:, 0] > 0).all()) and bool((t[:, 1] > 0).all()) and bool((t[:, 2] == 0).all())
