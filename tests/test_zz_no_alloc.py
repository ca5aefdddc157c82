"""The entry point that allocates nothing (bitlinear_forward_noalloc) against
bitlinear_forward with a caller workspace, through the C ABI: two calls in a
row on the library's own scratch, the second with a smaller input, each equal
to the workspace entry point bit for bit (int32 sums and fp32 outputs); a shape
past the scratch limit is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from ternary_weight_bitlinear_w1_amd import bitlinear as bl
from ternary_weight_bitlinear_w1_amd import synth

from _cases import Matrix, assert_equal, note, seed

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _case(m, n, k, segs, tag, codes_in=False):
    mats = [Matrix(s, k, seed(20, tag, i)) for i, s in enumerate(segs)]
    packed = []
    for mt in mats:
        p, _ = bl.quantize_weights(gpu(mt.w), gamma_in=gpu(np.array([mt.gamma])))
        packed.append(p)
    packed = torch.cat(packed) if len(packed) > 1 else packed[0]
    gam = [float(np.float32(mt.gamma)) for mt in mats]
    ends = list(np.cumsum(segs))
    x = gpu(synth.activations(seed(20, tag, 9), m, k, max(1, round(0.01 * k))))
    kw = {"x": x}
    if codes_in:
        c, d, _ = bl.quantize_acts(x)
        kw = {"codes": c, "deq": d}
    return packed, gam, ends, kw


@pytest.mark.parametrize("codes_in", [False, True])
def test_noalloc_matches_workspace_entry_point(codes_in):
    # 64 tokens of the down projection (split K: partial sums in the scratch),
    # then 3 tokens of q|k|v (the decode contraction), on the same scratch
    for (m, n, k, segs, tag) in [(64, 2560, 6912, [2560], 1), (3, 3840, 2560, [2560, 640, 640], 2)]:
        note(f"noalloc forward m={m} n={n} k={k} codes_in={codes_in}")
        packed, gam, ends, kw = _case(m, n, k, segs, tag, codes_in)
        y_ref, a_ref = bl.forward(packed, k, gam, ends, want_acc=True, **kw)
        y, a = bl.forward_noalloc(packed, k, gam, ends, want_acc=True, **kw)
        assert_equal(host(a), host(a_ref), f"acc m={m}")
        assert_equal(host(y).view(np.uint32), host(y_ref).view(np.uint32), f"y m={m}")


def test_noalloc_prefill_shape_and_limit():
    note("noalloc forward prefill M=4096 gate|up, then past the limit")
    m, k, segs = 4096, 2560, [6912, 6912]
    packed, gam, ends, kw = _case(m, sum(segs), k, segs, 3)
    y_ref = bl.forward(packed, k, gam, ends, **kw)
    y = bl.forward_noalloc(packed, k, gam, ends, **kw)
    assert_equal(host(y).view(np.uint32), host(y_ref).view(np.uint32), "y prefill")
    limit = bl.lib().bitlinear_forward_noalloc_max_scratch_bytes()
    assert limit == 32 << 20
    big_m = limit // 6912 + 1  # codes of big_m x 6912 bytes alone exceed the scratch
    g = (ctypes.c_float * 1)(1.0)
    se = (ctypes.c_int64 * 1)(2560)
    st = bl.lib().bitlinear_forward_noalloc(0x100000, None, None, None, big_m, 6912, 0x100000, 2560, g, se, 1,
                                            0x100000, None, 0, None)
    assert st == bl.ERR_WORKSPACE
    assert b"32 MiB" in bl.lib().bitlinear_last_error()
