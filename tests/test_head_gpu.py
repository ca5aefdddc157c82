"""The model's ends on the GPU against the CPU oracle: the embedding gather, and
the final norm (bfloat16 output, bit for bit) followed by the bfloat16 head
(logits within the fp32 summation bound k 2^-24 sum_k |o_k w[n][k]| of the
oracle's exact sum, reading R20)."""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_bitlinear_w1_amd import bitlinear as bl
from ternary_weight_bitlinear_w1_amd import synth

from _cases import assert_equal, note, seed

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
VOCAB, HIDDEN = 128256, 2560


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def head_table(sd, n, k):
    return oracle.round_bf16(synth.weights(sd, n, k, 0.02))


def check_logits(got, o, w, rows=None, what=""):
    sel = slice(None) if rows is None else rows
    ref, mag = oracle.lm_head(o, w if rows is None else w[rows])
    g = got[:, sel]
    k = o.shape[1]
    bound = k * 2.0 ** -24 * mag
    err = np.abs(g.astype(np.float64) - ref.astype(np.float64))
    assert (err <= bound).all(), f"{what}: max err / bound {np.max(err / np.maximum(bound, 1e-300)):.3f}"
    return ref


def test_embed():
    note("embed")
    table = head_table(seed(30, 0, 1), 1000, 256)
    ids = np.array([0, 999, 17, -1, 1000, 512, 17], dtype=np.int64)
    x = host(bl.embed(gpu(ids), gpu(table)))
    want = np.zeros((len(ids), 256), dtype=np.float32)
    ok = (ids >= 0) & (ids < 1000)
    want[ok] = oracle.bf16_to_f32(table[ids[ok]])
    assert_equal(x, want, "embedded rows")


# (m, k, n, scale): one to five tokens (five takes two passes over the head); k with a
# partial 512-column chunk and the widest k; a residual stream of large norm
CASES = [(1, 2560, 1000, 1.0), (3, 2560, 777, 1.0), (4, 128, 50, 1.0), (5, 2560, 300, 1.0), (2, 4096, 64, 1.0),
         (1, 40, 33, 1.0), (4, 2560, 4099, 2.0e4)]


@pytest.mark.parametrize("m,k,n,scale", CASES)
def test_lm_head(m, k, n, scale):
    note(f"lm_head m={m} k={k} n={n}")
    x = (scale * synth.activations(seed(31, m, k), m, k, synth.outlier_count(k))).astype(np.float32)
    g = (0.1 * (1.0 + 0.1 * synth.normal_f32(seed(31, 1, k), k))).astype(np.float32)
    w = head_table(seed(31, n, k), n, k)
    y, o = bl.lm_head(gpu(x), gpu(w), gain=gpu(g), want_normed=True)
    o_ref = oracle.final_norm(x, g)
    assert_equal(host(o).view(np.uint16), o_ref, "normed bfloat16")
    check_logits(host(y), o_ref, w, what="logits")
    # without the normed trace (the workspace holds it), and without a gain
    y2 = bl.lm_head(gpu(x), gpu(w), gain=gpu(g))
    assert_equal(host(y2), host(y), "logits through the workspace")
    y3 = bl.lm_head(gpu(x), gpu(w))
    check_logits(host(y3), oracle.final_norm(x, None), w, what="logits, gain 1")


@pytest.mark.parametrize("m", [1, 4])
def test_lm_head_full_size(m):
    """The 2B4T head (128256 x 2560): every normed value, and 3000 sampled logits
    rows (plus the first and last) of every token."""
    note(f"lm_head full size m={m}")
    x = (3.0e4 * synth.activations(seed(32, m, 1), m, HIDDEN)).astype(np.float32)
    g = np.full(HIDDEN, 0.1, dtype=np.float32)
    w = head_table(seed(32, 0, 2), VOCAB, HIDDEN)
    wg = gpu(w)
    y, o = bl.lm_head(gpu(x), wg, gain=gpu(g), want_normed=True)
    o_ref = oracle.final_norm(x, g)
    assert_equal(host(o).view(np.uint16), o_ref, "normed bfloat16")
    rows = np.unique(np.concatenate([[0, VOCAB - 1], np.random.default_rng(3).integers(0, VOCAB, 3000)]))
    check_logits(host(y), o_ref, w, rows=rows, what="sampled logits")
    y2 = bl.lm_head(gpu(x), wg, gain=gpu(g))
    assert_equal(host(y2), host(y), "repeat")
