"""Run-to-run determinism on the GPU: each workload runs three times on the same
inputs and must give the same bits every time. Where the oracle comparison is
bit-exact this follows from parity; here it is checked directly, also where the
comparison has a tolerance (the fp32 stack output after 30-layer-style chains,
the cached decoder's attention, the bfloat16 head). Every reduction on the
path has a fixed order (integer sums, fixed-order fp64 and fp32 trees); none
uses floating-point atomics.
"""
import copy

import numpy as np
import pytest
import torch

import oracle
from ternary_weight_bitlinear_w1_amd import bitlinear as bl
from ternary_weight_bitlinear_w1_amd import synth

from _cases import EPS, Matrix, assert_equal, note, seed
from test_block_gpu import _decoder_layer_mats, _gpu_layer, pack

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RUNS = 3


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _same(outs, what):
    for i, o in enumerate(outs[1:], 1):
        assert_equal(_bits(o), _bits(outs[0]), f"{what}: run {i} vs run 0")


def test_ffn_block_repeats():
    """The FFN block at M = 1024, hidden 512, intermediate 2048."""
    m, hdim, inter = 1024, 512, 2048
    note("determinism: FFN block m=1024")
    gate, up, down = (Matrix(inter, hdim, seed(40, 0, 1)), Matrix(inter, hdim, seed(40, 0, 2)),
                      Matrix(hdim, inter, seed(40, 0, 3)))
    spec = bl.BlockSpec(bl.BLOCK_FFN, hdim, inter,
                        [bl.LayerWeights(gate_up=pack([gate, up]),
                                         gate_up_gamma=[float(np.float32(gate.gamma)), float(np.float32(up.gamma))],
                                         down=pack([down]), down_gamma=float(np.float32(down.gamma)))], eps=EPS)
    x = gpu(synth.activations(seed(40, m, 5), m, hdim))
    _same([host(bl.block_forward(spec, x)) for _ in range(RUNS)], "FFN block")


@pytest.mark.parametrize("m", [1, 4, 64])
def test_decoder_stack_repeats(m):
    """Three layers at the 2B4T widths (H 2560, I 6912, 20 / 5 heads of 128): the
    fused one-token form, the 2-16-token chain and the 64-token chain with split
    K and K groups."""
    hdim, inter, nh, nkv, hd, layers = 2560, 6912, 20, 5, 128, 3
    note(f"determinism: decoder stack m={m}")
    layer_w = [_gpu_layer(_decoder_layer_mats(41, l, hdim, inter, nkv * hd), None) for l in range(layers)]
    spec = bl.BlockSpec(bl.BLOCK_DECODER, hdim, inter, layer_w, nh, nkv, hd, EPS)
    x = gpu(synth.activations(seed(41, m, 5), m, hdim, 26))
    _same([host(bl.block_forward(spec, x)) for _ in range(RUNS)], f"stack m={m}")


@pytest.mark.parametrize("positions", [[4095], [4095, 17, 2048, 1000]])
def test_cached_decoder_and_head_repeats(positions):
    """Two cached decoder layers at the 2B4T widths over a 4096-position context
    (RoPE, cache append, causal attention), then the final norm and a bfloat16
    head of 4096 rows. Each run starts from the same caches; the caches after the
    step must match as well."""
    hdim, inter, nh, nkv, hd, layers, tmax, vocab = 2560, 6912, 20, 5, 128, 2, 4096, 4096
    m = len(positions)
    note(f"determinism: cached decoder + head m={m}")
    r = np.random.default_rng(42 + m)
    slot = np.arange(m, dtype=np.int64)
    pos = np.array(positions, dtype=np.int64)
    layer_w = [_gpu_layer(_decoder_layer_mats(42, l, hdim, inter, nkv * hd), None) for l in range(layers)]
    caches = [(oracle.round_bf16(r.normal(size=(m, nkv, tmax, hd)).astype(np.float32)),
               oracle.round_bf16(r.normal(size=(m, nkv, tmax, hd)).astype(np.float32))) for _ in range(layers)]
    table = bl.rope_table(5e5, hd, tmax, DEV)
    head = gpu(oracle.round_bf16(synth.weights(seed(42, 0, 50), vocab, hdim, 0.02)))
    gain = gpu(np.full(hdim, 1.0, dtype=np.float32))
    x = gpu(synth.activations(seed(42, m, 5), m, hdim, 26))
    outs, logits, kcs = [], [], []
    for _ in range(RUNS):
        lws = []
        for lw, (kc, vc) in zip(layer_w, caches):
            c = copy.copy(lw)
            c.k_cache, c.v_cache = gpu(kc), gpu(vc)
            lws.append(c)
        spec = bl.BlockSpec(bl.BLOCK_DECODER_CACHED, hdim, inter, lws, nh, nkv, hd, EPS, slot=gpu(slot),
                            pos=gpu(pos), rope_table=table)
        y = bl.block_forward(spec, x)
        outs.append(host(y))
        logits.append(host(bl.lm_head(y, head, gain, EPS)))
        kcs.append(np.concatenate([host(c.k_cache).view(np.uint16).ravel() for c in lws]))
    _same(outs, "cached decoder output")
    _same(logits, "head logits")
    _same(kcs, "key caches after the step")
