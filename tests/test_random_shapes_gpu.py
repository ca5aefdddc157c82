"""Seeded random shapes through every contraction entry point, against the CPU
oracle element by element: the kernel choice depends on m, n, k (decode dot
product, decode MFMA, fused decode, pipelined GEMM with and without split K,
small tiles, the generic GEMM, the gated GEMM), so random shapes reach
combinations the listed cases do not. The shapes come from a fixed seed and
are printed before each case."""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_bitlinear_w1_amd import bitlinear as bl
from ternary_weight_bitlinear_w1_amd import synth

from _cases import EPS, Matrix, assert_equal, assert_rel, note, seed, stacked

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _shapes(count, seed_value):
    rng = np.random.default_rng(seed_value)
    out = []
    for _ in range(count):
        m = int(rng.choice([1, 2, 3, 4, 5, 16, 17, 33, 64, 65, 100, 129, 200, 300]))
        k = int(16 * rng.integers(1, 160))        # up to 2544
        if rng.random() < 0.5:
            k = 128 * int(rng.integers(1, 20))    # pipelined kernels need k % 128 == 0
        n = int(rng.choice([16 * rng.integers(1, 64), 64 * rng.integers(1, 40), 256 * rng.integers(1, 10)]))
        out.append((m, n, k))
    return out


FORWARD = _shapes(24, 20260101)


@pytest.mark.parametrize("m,n,k", FORWARD)
def test_random_forward(m, n, k):
    note(f"random forward m={m} n={n} k={k}")
    cut = max(16, (n // 3) // 16 * 16) if n >= 48 else n
    mats = [Matrix(cut, k, seed(10, n, k))] + ([Matrix(n - cut, k, seed(10, n, k + 1))] if cut < n else [])
    codes, gammas, ends = stacked(mats)
    packed = torch.cat([bl.quantize_weights(gpu(mt.w), gamma_in=gpu(np.array([mt.gamma])))[0] for mt in mats])
    x = synth.activations(seed(10, m, k), m, k, 1 if k >= 100 else 0)
    g = [float(np.float32(v)) for v in gammas]
    ref = oracle.forward(x, codes, gammas, ends)
    for path in [bl.PATH_AUTO, bl.PATH_PREFILL] + ([bl.PATH_DECODE] if m <= 16 else []):
        y, acc = bl.forward(packed, k, g, ends, x=gpu(x), want_acc=True, path=path)
        assert_equal(host(acc), ref["acc"], f"acc path {path}")
        assert_equal(host(y), ref["y"], f"y path {path}")


GLU = [(m, 4 * max(1, n // 8), k) for m, n, k in _shapes(10, 20260202)] + [(65, 128, 1280), (300, 384, 256)]


@pytest.mark.parametrize("m,inter,k", GLU)
def test_random_relu2_glu(m, inter, k):
    note(f"random relu2 glu m={m} inter={inter} k={k}")
    mats = [Matrix(inter, k, seed(11, inter, 1)), Matrix(inter, k, seed(11, inter, 2))]
    codes, gammas, ends = stacked(mats)
    packed = torch.cat([bl.quantize_weights(gpu(mt.w), gamma_in=gpu(np.array([mt.gamma])))[0] for mt in mats])
    x = synth.activations(seed(11, m, k), m, k, 1 if k >= 100 else 0)
    ref = oracle.relu2_mul(oracle.forward(x, codes, gammas, ends)["y"], inter)
    y = bl.forward_relu2_glu(packed, k, [float(np.float32(v)) for v in gammas], x=gpu(x))
    assert_equal(host(y), ref, "gated y")


FFN = [(1, 64, 128), (3, 128, 192), (4, 256, 512), (7, 64, 192), (70, 128, 256), (130, 256, 384), (2, 512, 1024)]


@pytest.mark.parametrize("m,hdim,inter", FFN)
def test_random_ffn_block(m, hdim, inter):
    """FFN block chain with a random ffn_sub_norm gain: fused decode form (m <= 4),
    quantize + contraction chain, gated GEMM (m > 64)."""
    note(f"random ffn block m={m} H={hdim} I={inter}")
    gate, up, down = Matrix(inter, hdim, seed(12, m, 1)), Matrix(inter, hdim, seed(12, m, 2)), \
        Matrix(hdim, inter, seed(12, m, 3))
    gain = (1.0 + 0.1 * synth.normal_f32(seed(12, m, 4), inter)).astype(np.float32)
    pack = lambda mats: torch.cat([bl.quantize_weights(gpu(mt.w), gamma_in=gpu(np.array([mt.gamma])))[0]
                                   for mt in mats])
    spec = bl.BlockSpec(bl.BLOCK_FFN, hdim, inter,
                        [bl.LayerWeights(gate_up=pack([gate, up]),
                                         gate_up_gamma=[float(np.float32(gate.gamma)), float(np.float32(up.gamma))],
                                         down=pack([down]), down_gamma=float(np.float32(down.gamma)),
                                         ffn_sub_norm_gain=gpu(gain))], eps=EPS)
    x = synth.activations(seed(12, m, 5), m, hdim, 1)
    ref = oracle.ffn_block(x, np.concatenate([gate.codes, up.codes]), [gate.gamma, up.gamma], down.codes,
                           down.gamma, gain, EPS)
    assert_rel(host(bl.block_forward(spec, gpu(x))), ref["y"], what="ffn y")
