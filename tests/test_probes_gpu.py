"""The measurement probes run on the GPU and leave their sink alone (they
compute nothing a caller uses; the sink is written only on a chance match of
the folded value with a fixed key, which these inputs do not give)."""
import pytest
import torch

from ternary_weight_bitlinear_w1_amd import bitlinear as bl

from _cases import note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_probe_read_runs():
    note("probe read: 4 MiB, default and fixed grids")
    buf = torch.zeros(1 << 20, dtype=torch.float32, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    for grid in (0, 7, 256):
        bl.probe_read(buf, grid=grid, sink=sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0


@pytest.mark.parametrize("varied", [False, True])
def test_probe_mfma_runs(varied):
    note(f"probe mfma varied={varied}")
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    bl.probe_mfma(10, 512, sink, varied=varied)
    torch.cuda.synchronize()
