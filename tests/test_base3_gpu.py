"""Five codes per byte (reading R18) on the GPU against the CPU oracle.

The repacking kernel must give the oracle's base-3 bytes exactly, from the
oracle's two-bit bytes; the 1..4-token contraction over base-3 weights must give
the oracle's int32 sums and fp32 outputs bit for bit, and the same result as the
two-bit path on the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_bitlinear_w1_amd import bitlinear as bl
from ternary_weight_bitlinear_w1_amd import synth

from _cases import Matrix, assert_equal, note, seed, stacked

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("n,k", [(1, 16), (3, 48), (5, 80), (7, 96), (17, 272), (640, 2560), (2560, 6912),
                                 (33, 8192), (9, 4112)])
def test_pack_base3_matches_oracle(n, k):
    note(f"pack_base3 n={n} k={k}")
    r = np.random.default_rng(seed(20, n, k))
    c = r.integers(-1, 2, size=(n, k)).astype(np.int8)
    two_bit = oracle.pack(c)
    w3 = bl.pack_base3(gpu(two_bit), k)
    assert tuple(w3.shape) == (n, oracle.base3_row_bytes(k))
    assert_equal(host(w3), oracle.pack_base3(c), "base-3 bytes")


def test_pack_base3_invalid_field_reads_as_zero():
    """A two-bit field of 3 is no code; the repacking takes it as code 0, as the
    oracle's unpacking does."""
    note("pack_base3 invalid fields")
    r = np.random.default_rng(7)
    p = r.integers(0, 256, size=(40, 64), dtype=np.uint8)  # k = 256, many fields of 3
    codes, bad = oracle.unpack(p, 256)
    assert bad > 0
    assert_equal(host(bl.pack_base3(gpu(p), 256)), oracle.pack_base3(codes), "base-3 bytes")


# (m, n, k, segments): rows not a multiple of 8; K from one 80-code block to 8192, not a multiple of 80;
# every split of K over waves (n / 32 >= 256: one wave per row group; n / 16 >= 256: two; else four)
CASES = [(1, 40, 48, 1), (2, 200, 80, 1), (3, 1000, 576, 2), (4, 77, 8192, 1), (1, 9000, 1024, 2),
         (4, 5000, 448, 1), (3, 33, 4112, 1), (2, 4100, 6912, 2), (1, 13824, 2560, 2), (4, 13824, 2560, 2),
         (1, 2560, 6912, 1), (4, 2560, 6912, 1)]


@pytest.mark.parametrize("m,n,k,segs", CASES)
def test_forward_base3(m, n, k, segs):
    note(f"forward_base3 m={m} n={n} k={k}")
    n1 = n // 2 if segs == 2 else n
    mats = [Matrix(n1, k, seed(21, n, 1))] + ([Matrix(n - n1, k, seed(21, n, 2), sigma=0.05)] if segs == 2 else [])
    codes, gammas, ends = stacked(mats)
    gf = [float(np.float32(g)) for g in gammas]
    x = synth.activations(seed(21, m, k), m, k, synth.outlier_count(k))
    ref = oracle.forward(x, codes, gammas, ends)
    w3 = gpu(oracle.pack_base3(codes))
    y, acc = bl.forward_base3(w3, k, gf, ends, x=gpu(x), want_acc=True)
    assert_equal(host(acc), ref["acc"], "acc")
    assert_equal(host(y), ref["y"], "y bit-exact")
    # codes given instead of x, weights repacked on the GPU from the two-bit bytes
    q, dq = oracle.quant_absmax(x)
    w3g = bl.pack_base3(gpu(oracle.pack(codes)), k)
    y2 = bl.forward_base3(w3g, k, gf, ends, codes=gpu(q), deq=gpu(dq))
    assert_equal(host(y2), ref["y"], "y from codes")
    # the two-bit path gives the same
    y3 = bl.forward(gpu(oracle.pack(codes)), k, gf, ends, x=gpu(x), path=bl.PATH_DECODE)
    assert_equal(host(y3), host(y), "two-bit path")


def test_forward_base3_invalid_bytes_read_as_zero():
    """Bytes 243..255 hold no codes: they contribute nothing, as the oracle's
    unpacking (five zero codes) says."""
    note("forward_base3 invalid bytes")
    m, n, k = 2, 64, 320
    r = np.random.default_rng(9)
    w3 = r.integers(0, 256, size=(n, oracle.base3_row_bytes(k)), dtype=np.uint8)
    codes, bad = oracle.unpack_base3(w3, k)
    assert bad > 0
    x = synth.activations(seed(22, m, k), m, k)
    ref = oracle.forward(x, codes, [0.03], [n])
    y, acc = bl.forward_base3(gpu(w3), k, [float(np.float32(0.03))], [n], x=gpu(x), want_acc=True)
    assert_equal(host(acc), ref["acc"], "acc")
    assert_equal(host(y), ref["y"], "y")


def test_forward_base3_empty_and_zero_rows():
    """m = 0 is a no-op; an all-zero token gives zeros."""
    note("forward_base3 m=0 and zero rows")
    n, k = 96, 160
    mats = [Matrix(n, k, seed(23, 0, 1))]
    codes, gammas, ends = stacked(mats)
    w3 = gpu(oracle.pack_base3(codes))
    y0 = bl.forward_base3(w3, k, [float(np.float32(gammas[0]))], ends, x=torch.empty((0, k), device=DEV))
    assert tuple(y0.shape) == (0, n)
    x = np.zeros((3, k), dtype=np.float32)
    x[1] = synth.activations(seed(23, 1, 2), 1, k)[0]
    ref = oracle.forward(x, codes, gammas, ends)
    y = bl.forward_base3(w3, k, [float(np.float32(gammas[0]))], ends, x=gpu(x))
    assert_equal(host(y), ref["y"], "y")
    assert not host(y)[0].any() and not host(y)[2].any()
