"""Block chains on the GPU against the CPU oracle, free running from the same
seeded inputs (the oracle never sees a GPU value).

FFN block: x -> int8 codes -> gate|up -> ReLU^2 -> ffn_sub_norm -> down, at
hidden 512 / intermediate 2048 and M = 1024 (and at decode sizes).
Decoder stack: the projections of n_layers blocks in the order of the nnterp
page's "The block, in order", attention taken for tokens that attend only to
themselves; 30 layers at the 2B4T shapes (M = 1, and sampled tokens of M = 64;
tokens are independent, so the oracle computes only the sampled rows).
"""
import copy

import numpy as np
import pytest
import torch

import oracle
from ternary_weight_bitlinear_w1_amd import bitlinear as bl
from ternary_weight_bitlinear_w1_amd import synth

from _cases import EPS, Matrix, assert_equal, assert_rel, note, seed

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def pack(mats):
    parts = [bl.quantize_weights(gpu(m.w), gamma_in=gpu(np.array([m.gamma])))[0] for m in mats]
    return torch.cat(parts) if len(parts) > 1 else parts[0]


def f32(g):
    return float(np.float32(g))


# ------------------------------------------------------------------------------ FFN block
@pytest.mark.parametrize("m", [1024, 16, 1, 37, 2, 3, 4, 5])
def test_ffn_block(m):
    hdim, inter = 512, 2048
    note(f"block FFN m={m} H={hdim} I={inter}")
    gate = Matrix(inter, hdim, seed(2, 0, 1))
    up = Matrix(inter, hdim, seed(2, 0, 2))
    down = Matrix(hdim, inter, seed(2, 0, 3))
    x = synth.activations(seed(2, m, 5), m, hdim)
    spec = bl.BlockSpec(bl.BLOCK_FFN, hdim, inter,
                        [bl.LayerWeights(gate_up=pack([gate, up]), gate_up_gamma=[f32(gate.gamma), f32(up.gamma)],
                                         down=pack([down]), down_gamma=f32(down.gamma))], eps=EPS)
    tr = {"codes_in": torch.empty((m, hdim), dtype=torch.int8, device=DEV),
          "codes_ffn": torch.empty((m, inter), dtype=torch.int8, device=DEV),
          "deq": torch.zeros((4, m), dtype=torch.float32, device=DEV),
          "gate_up": torch.empty((m, 2 * inter), dtype=torch.float32, device=DEV),
          "acc_gate_up": torch.empty((m, 2 * inter), dtype=torch.int32, device=DEV),
          "acc_down": torch.empty((m, hdim), dtype=torch.int32, device=DEV)}
    y = bl.block_forward(spec, gpu(x), trace=tr)
    ref = oracle.ffn_block(x, np.concatenate([gate.codes, up.codes]), [gate.gamma, up.gamma], down.codes,
                           down.gamma, None, EPS)
    assert_equal(host(tr["codes_in"]), ref["q1"], "input codes")
    assert_equal(host(tr["acc_gate_up"]), ref["acc_gu"], "gate|up acc")
    assert_equal(host(tr["gate_up"]), ref["gu"], "gate|up")
    assert_equal(host(tr["codes_ffn"]), ref["q2"], "ffn_sub_norm codes")
    assert_rel(host(tr["deq"])[3], ref["deq2"], what="ffn_sub_norm deq")
    assert_equal(host(tr["acc_down"]), ref["acc_down"], "down acc")
    assert_rel(host(y), ref["y"], what="y")
    assert_equal(host(bl.block_forward(spec, gpu(x))), host(y), "untraced y")


# ------------------------------------------------------------------------------ decoder stack
def _decoder_layer_mats(cfg, layer, hdim, inter, kvd):
    names = [("q", hdim, hdim), ("k", kvd, hdim), ("v", kvd, hdim), ("o", hdim, hdim), ("gate", inter, hdim),
             ("up", inter, hdim), ("down", hdim, inter)]
    return {nm: Matrix(n, k, seed(cfg, layer, 10 + i)) for i, (nm, n, k) in enumerate(names)}


def _oracle_weights(mt, gains):
    w = {"qkv": np.concatenate([mt["q"].codes, mt["k"].codes, mt["v"].codes]),
         "g_qkv": [mt["q"].gamma, mt["k"].gamma, mt["v"].gamma], "o": mt["o"].codes, "g_o": mt["o"].gamma,
         "gu": np.concatenate([mt["gate"].codes, mt["up"].codes]), "g_gu": [mt["gate"].gamma, mt["up"].gamma],
         "down": mt["down"].codes, "g_down": mt["down"].gamma}
    if gains is not None:
        w.update(gains)
    return w


def _gpu_layer(mt, gains):
    lw = bl.LayerWeights(qkv=pack([mt["q"], mt["k"], mt["v"]]),
                         qkv_gamma=[f32(mt["q"].gamma), f32(mt["k"].gamma), f32(mt["v"].gamma)],
                         o=pack([mt["o"]]), o_gamma=f32(mt["o"].gamma), gate_up=pack([mt["gate"], mt["up"]]),
                         gate_up_gamma=[f32(mt["gate"].gamma), f32(mt["up"].gamma)], down=pack([mt["down"]]),
                         down_gamma=f32(mt["down"].gamma))
    if gains is not None:
        lw.input_norm_gain = gpu(gains["n_in"])
        lw.attn_sub_norm_gain = gpu(gains["n_attn"])
        lw.post_attn_norm_gain = gpu(gains["n_post"])
        lw.ffn_sub_norm_gain = gpu(gains["n_ffn"])
    return lw


def _trace(L, m, hdim, inter, q):
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt, device=DEV)
    return {"codes_in": z(L, m, hdim, dt=torch.int8), "codes_attn": z(L, m, hdim, dt=torch.int8),
            "codes_post": z(L, m, hdim, dt=torch.int8), "codes_ffn": z(L, m, inter, dt=torch.int8),
            "deq": z(L, 4, m), "qkv": z(L, m, q), "h": z(L, m, hdim), "gate_up": z(L, m, 2 * inter),
            "x_out": z(L, m, hdim), "acc_qkv": z(L, m, q, dt=torch.int32), "acc_o": z(L, m, hdim, dt=torch.int32),
            "acc_gate_up": z(L, m, 2 * inter, dt=torch.int32), "acc_down": z(L, m, hdim, dt=torch.int32)}


def _compare_layer(tr, l, ref, rows=None):
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    g = {k: host(v[l]) for k, v in tr.items()}
    assert_equal(sel(g["codes_in"]), ref["qkv"]["q"], f"layer {l} input codes")
    assert_equal(sel(g["acc_qkv"]), ref["qkv"]["acc"], f"layer {l} qkv acc")
    assert_equal(sel(g["qkv"]), ref["qkv"]["y"], f"layer {l} qkv")
    assert_equal(sel(g["codes_attn"]), ref["o"]["q"], f"layer {l} attn_sub_norm codes")
    assert_equal(sel(g["acc_o"]), ref["o"]["acc"], f"layer {l} o acc")
    assert_equal(sel(g["h"]), ref["h"], f"layer {l} h")
    assert_equal(sel(g["codes_post"]), ref["gu"]["q"], f"layer {l} post-norm codes")
    assert_equal(sel(g["acc_gate_up"]), ref["gu"]["acc"], f"layer {l} gate|up acc")
    assert_equal(sel(g["codes_ffn"]), ref["down"]["q"], f"layer {l} ffn_sub_norm codes")
    assert_equal(sel(g["acc_down"]), ref["down"]["acc"], f"layer {l} down acc")
    deq = g["deq"] if rows is None else g["deq"][:, rows]
    for j, st in enumerate(("qkv", "o", "gu", "down")):
        assert_rel(deq[j], ref[st]["deq"], what=f"layer {l} deq {st}")
    assert_rel(sel(g["x_out"]), ref["x"], what=f"layer {l} output")


@pytest.mark.parametrize("m,layers", [(5, 3), (20, 2), (1, 2)])
def test_decoder_stack_small(m, layers):
    """Small dims with random gains: H=64 (8 heads of 8), 2 kv heads, I=96."""
    hdim, inter, nh, nkv, hd = 64, 96, 8, 2, 8
    note(f"block decoder small m={m} layers={layers}")
    kvd = nkv * hd
    x = synth.activations(seed(6, m, 5), m, hdim, 1)
    gpu_layers, refs = [], []
    xo = x
    for l in range(layers):
        mt = _decoder_layer_mats(6, l, hdim, inter, kvd)
        gains = {nm: (1.0 + 0.1 * synth.normal_f32(seed(6, l, 30 + i), n)).astype(np.float32)
                 for i, (nm, n) in enumerate((("n_in", hdim), ("n_attn", hdim), ("n_post", hdim), ("n_ffn", inter)))}
        ref = oracle.decoder_layer(xo, _oracle_weights(mt, gains), EPS, nh, nkv, hd)
        refs.append(ref)
        xo = ref["x"]
        gpu_layers.append(_gpu_layer(mt, gains))
    spec = bl.BlockSpec(bl.BLOCK_DECODER, hdim, inter, gpu_layers, nh, nkv, hd, EPS)
    tr = _trace(layers, m, hdim, inter, hdim + 2 * kvd)
    y = bl.block_forward(spec, gpu(x), trace=tr)
    for l in range(layers):
        _compare_layer(tr, l, refs[l])
    assert_rel(host(y), xo, what="stack output")


@pytest.mark.parametrize("m,layers", [(1, 3), (2, 2), (3, 2), (4, 2), (5, 2)])
def test_decoder_stack_fused_sizes(m, layers):
    """Dims that the one-launch-per-projection decode form takes (every
    projection input a multiple of 64; m <= 2), random gains: H=128 (8 heads
    of 16), 2 kv heads, I=192. m = 3 to 5 take the quantize -> contract chain."""
    hdim, inter, nh, nkv, hd = 128, 192, 8, 2, 16
    note(f"block decoder fused sizes m={m} layers={layers}")
    kvd = nkv * hd
    x = synth.activations(seed(7, m, 5), m, hdim, 2)
    gpu_layers, refs = [], []
    xo = x
    for l in range(layers):
        mt = _decoder_layer_mats(7, l, hdim, inter, kvd)
        gains = {nm: (1.0 + 0.1 * synth.normal_f32(seed(7, l, 30 + i), n)).astype(np.float32)
                 for i, (nm, n) in enumerate((("n_in", hdim), ("n_attn", hdim), ("n_post", hdim), ("n_ffn", inter)))}
        ref = oracle.decoder_layer(xo, _oracle_weights(mt, gains), EPS, nh, nkv, hd)
        refs.append(ref)
        xo = ref["x"]
        gpu_layers.append(_gpu_layer(mt, gains))
    spec = bl.BlockSpec(bl.BLOCK_DECODER, hdim, inter, gpu_layers, nh, nkv, hd, EPS)
    tr = _trace(layers, m, hdim, inter, hdim + 2 * kvd)
    y = bl.block_forward(spec, gpu(x), trace=tr)
    for l in range(layers):
        _compare_layer(tr, l, refs[l])
    assert_rel(host(y), xo, what="stack output")
    y2 = bl.block_forward(spec, gpu(x))  # no trace: the scratch buffers carry the chain
    assert_equal(host(y2), host(y), "untraced output")


@pytest.mark.parametrize("m,hdim,inter,nh,nkv,hd", [(24, 768, 1024, 12, 4, 64), (17, 2048, 1024, 16, 4, 128)])
def test_decoder_stack_split_chain(m, hdim, inter, nh, nkv, hd):
    """17 <= m <= 64 at dims where every projection splits K (2 ways at the
    first shape; 4 ways for q|k|v, o and gate|up and 2 for down at the second):
    without a trace the quantizations read the split partial sums themselves and
    the last down projection is finished into the residual sum. Layer 0 has
    random gains, layer 1 none (gain 1). Traced run against the oracle, then the
    untraced run bit-equal to the traced one."""
    layers = 2
    note(f"block decoder split chain m={m} H={hdim} I={inter}")
    kvd = nkv * hd
    x = synth.activations(seed(8, m, 5), m, hdim, 1)
    gpu_layers, refs = [], []
    xo = x
    for l in range(layers):
        mt = _decoder_layer_mats(8, l, hdim, inter, kvd)
        gains = None
        if l == 0:
            gains = {nm: (1.0 + 0.1 * synth.normal_f32(seed(8, l, 30 + i), n)).astype(np.float32)
                     for i, (nm, n) in enumerate((("n_in", hdim), ("n_attn", hdim), ("n_post", hdim),
                                                  ("n_ffn", inter)))}
        ref = oracle.decoder_layer(xo, _oracle_weights(mt, gains), EPS, nh, nkv, hd)
        refs.append(ref)
        xo = ref["x"]
        gpu_layers.append(_gpu_layer(mt, gains))
    spec = bl.BlockSpec(bl.BLOCK_DECODER, hdim, inter, gpu_layers, nh, nkv, hd, EPS)
    tr = _trace(layers, m, hdim, inter, hdim + 2 * kvd)
    y = bl.block_forward(spec, gpu(x), trace=tr)
    for l in range(layers):
        _compare_layer(tr, l, refs[l])
    assert_rel(host(y), xo, what="stack output")
    y2 = bl.block_forward(spec, gpu(x))
    assert_equal(host(y2), host(y), "untraced output")


def test_decoder_stack_30_layers():
    """30 layers at the 2B4T shapes (H 2560, I 6912, 20 / 5 heads of 128, gains 1):
    M = 1 in full, and 3 sampled tokens of M = 64, all from the same weights. At
    M = 64 every projection but gate|up splits K; the traced run is compared
    stage by stage on the sampled tokens (codes and int32 sums bit-exact), and
    the untraced run, whose quantizations read the split partial sums, must give
    the traced output bit for bit."""
    hdim, inter, nh, nkv, hd, layers = 2560, 6912, 20, 5, 128, 30
    kvd = nkv * hd
    note("block decoder 30 layers, M=1 and M=64")
    x1 = synth.activations(seed(5, 1, 5), 1, hdim)
    x64 = synth.activations(seed(5, 64, 5), 64, hdim)
    samples = np.array([0, 37, 63])
    xo = np.concatenate([x1, x64[samples]])
    gpu_layers, refs = [], []
    for l in range(layers):
        mt = _decoder_layer_mats(5, l, hdim, inter, kvd)
        gpu_layers.append(_gpu_layer(mt, None))
        ref = oracle.decoder_layer(xo, _oracle_weights(mt, None), EPS, nh, nkv, hd)
        refs.append(ref)
        xo = ref["x"]
        del mt
    spec = bl.BlockSpec(bl.BLOCK_DECODER, hdim, inter, gpu_layers, nh, nkv, hd, EPS)
    tr = _trace(layers, 1, hdim, inter, hdim + 2 * kvd)
    y1 = bl.block_forward(spec, gpu(x1), trace=tr)
    for l in range(layers):
        _compare_layer(tr, l, {k: _rows(v, [0]) for k, v in refs[l].items()})
    assert_rel(host(y1), xo[:1], what="M=1 output")
    del tr
    tr64 = _trace(layers, 64, hdim, inter, hdim + 2 * kvd)
    y64t = bl.block_forward(spec, gpu(x64), trace=tr64)
    for l in range(layers):
        _compare_layer(tr64, l, {k: _rows(v, [1, 2, 3]) for k, v in refs[l].items()}, rows=samples)
    del tr64
    y64 = bl.block_forward(spec, gpu(x64))
    assert_equal(host(y64), host(y64t), "M=64 untraced output")
    assert_rel(host(y64)[samples], xo[1:], what="M=64 sampled outputs")


def _rows(v, rows):
    if isinstance(v, dict):
        return {k: _rows(a, rows) for k, a in v.items()}
    return v[rows]


# ------------------------------------------------------------------------------ decoder with a KV cache
def _attn_bound_ok(got, ref, vmag, smag, hd, tmax):
    S = (tmax + 255) // 256
    factor = 2.0 ** -24 * (2 * (hd + 1) * np.repeat(smag, hd, axis=1) + 2 * (192 + S))
    return np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= factor * vmag


# (hidden, intermediate, q heads, kv heads, layers, t_max, positions): the small layout above; a token whose
# position is past t_max (zeros from attention, nothing appended); groups of 1 and 8 q heads per kv head; the
# 2B4T layout (20 q heads on 5 kv heads) with one token (16 rows per workgroup) and two (8 rows)
ROPE_FUSED = [(512, 768, 4, 1, 2, 512, [5, 300]), (512, 768, 4, 1, 2, 512, [511]),
              (512, 768, 4, 1, 2, 512, [512, 77]), (512, 768, 4, 4, 1, 256, [100, 5]),
              (1024, 768, 8, 1, 1, 256, [255, 31]), (2560, 6912, 20, 5, 1, 512, [511]),
              (2560, 6912, 20, 5, 1, 1024, [1023, 64]),
              # 3 to 16 tokens: the decode contraction's RoPE form; 17 takes the separate kernel
              (512, 768, 4, 1, 2, 512, [0, 5, 300]), (512, 768, 4, 1, 2, 512, [3, 512, 77, 0]),
              (1024, 768, 8, 1, 1, 256, [255, 0, 31, 100, 7]), (512, 768, 4, 4, 1, 256, list(range(0, 160, 10))),
              (2560, 6912, 20, 5, 1, 1024, [1023, 64, 5, 900]), (512, 768, 4, 1, 1, 256, list(range(3, 255, 15)))]


@pytest.mark.parametrize("hdim,inter,nh,nkv,layers,tmax,positions", ROPE_FUSED)
def test_decoder_cached_rope_fused(hdim, inter, nh, nkv, layers, tmax, positions):
    _rope_fused_case(hdim, inter, nh, nkv, layers, tmax, positions, None)


# a token whose slot is outside the caches (no append, zeros from attention): one token, two (the fused
# decode form) and three (the decode contraction's RoPE form)
ROPE_FUSED_SLOTS = [(512, 768, 4, 1, 2, 512, [5], [3]), (512, 768, 4, 1, 2, 512, [5, 300], [1, -1]),
                    (512, 768, 4, 1, 2, 512, [0, 5, 300], [2, 7, 0])]


@pytest.mark.parametrize("hdim,inter,nh,nkv,layers,tmax,positions,slots", ROPE_FUSED_SLOTS)
def test_decoder_cached_rope_fused_bad_slot(hdim, inter, nh, nkv, layers, tmax, positions, slots):
    _rope_fused_case(hdim, inter, nh, nkv, layers, tmax, positions, slots)


def _rope_fused_case(hdim, inter, nh, nkv, layers, tmax, positions, slots):
    """Without a q|k|v trace the q|k|v projection takes RoPE and the cache
    append in its epilogue: the fused decode form for one or two tokens, the
    decode contraction for 3 to 16. Its output and both caches equal
    those of the traced run bit for bit (that run rotates and appends in a
    kernel of its own, and the test above checks its stages against the
    oracle), with no trace and with an attention trace alone."""
    hd, theta = 128, 5e5
    m = len(positions)
    note(f"block decoder cached, fused rope m={m} hidden={hdim}")
    kvd = nkv * hd
    Q = hdim + 2 * kvd
    r = np.random.default_rng(60 + m)
    slot = np.arange(m, dtype=np.int64)[::-1].copy() if slots is None else np.array(slots, dtype=np.int64)
    pos = np.array(positions, dtype=np.int64)
    x = synth.activations(seed(10, m, 5), m, hdim, 1)
    layers_w, caches0 = [], []
    for l in range(layers):
        mt = _decoder_layer_mats(10, l, hdim, inter, kvd)
        layers_w.append(_gpu_layer(mt, None))
        caches0.append((oracle.round_bf16(r.normal(size=(m, nkv, tmax, hd)).astype(np.float32)),
                        oracle.round_bf16(r.normal(size=(m, nkv, tmax, hd)).astype(np.float32))))

    def run(trace):
        lws = []
        for lw, (kc, vc) in zip(layers_w, caches0):
            c = copy.copy(lw)
            c.k_cache, c.v_cache = gpu(kc), gpu(vc)
            lws.append(c)
        spec = bl.BlockSpec(bl.BLOCK_DECODER_CACHED, hdim, inter, lws, nh, nkv, hd, EPS, slot=gpu(slot),
                            pos=gpu(pos), rope_table=bl.rope_table(theta, hd, 4096, DEV))
        y = host(bl.block_forward(spec, gpu(x), trace=trace))
        return y, [(host(c.k_cache), host(c.v_cache)) for c in lws]

    y_ref, c_ref = run(_trace(layers, m, hdim, inter, Q))
    att = torch.zeros((layers, m, hdim), dtype=torch.float32, device=DEV)
    for trace in (None, {"attn": att}):
        y, c = run(trace)
        assert_equal(y, y_ref, "block output")
        for l in range(layers):
            assert_equal(c[l][0].view(np.uint16), c_ref[l][0].view(np.uint16), f"layer {l} key cache")
            assert_equal(c[l][1].view(np.uint16), c_ref[l][1].view(np.uint16), f"layer {l} value cache")
    valid = (slot >= 0) & (slot < m) & (pos >= 0) & (pos < tmax)
    a = host(att)
    assert (not valid.any() or a[:, valid].any()) and not a[:, ~valid].any(), "attention: tokens in range only"


@pytest.mark.parametrize("positions", [[5, 300], [0, 1, 2, 100, 257, 511], [0, 7, 300]])
def test_decoder_cached_teacher_forced(positions):
    """Two decoder layers with RoPE, KV caches and causal attention (H = 512: 4
    query heads of 128 on 1 key/value head; I = 768). Two tokens take the
    fused decode form, three and six the quantize -> contract chain. Every stage is
    checked against the oracle fed the GPU's own input to that stage: ints
    bit-exact, the projections' fp32 outputs and both caches bit-exact, the
    attention within its fp32 bound."""
    hdim, inter, nh, nkv, hd, layers, tmax, theta = 512, 768, 4, 1, 128, 2, 512, 5e5
    m = len(positions)
    note(f"block decoder cached m={m}")
    kvd = nkv * hd
    Q = hdim + 2 * kvd
    r = np.random.default_rng(50 + m)
    slot = np.arange(m, dtype=np.int64)[::-1].copy()
    pos = np.array(positions, dtype=np.int64)
    x = synth.activations(seed(9, m, 5), m, hdim, 1)
    mats, gains, caches0, gpu_layers = [], [], [], []
    for l in range(layers):
        mt = _decoder_layer_mats(9, l, hdim, inter, kvd)
        g = None
        if l == 0:
            g = {nm: (1.0 + 0.1 * synth.normal_f32(seed(9, l, 30 + i), n)).astype(np.float32)
                 for i, (nm, n) in enumerate((("n_in", hdim), ("n_attn", hdim), ("n_post", hdim), ("n_ffn", inter)))}
        kc = oracle.round_bf16(r.normal(size=(m, nkv, tmax, hd)).astype(np.float32))
        vc = oracle.round_bf16(r.normal(size=(m, nkv, tmax, hd)).astype(np.float32))
        lw = _gpu_layer(mt, g)
        lw.k_cache, lw.v_cache = gpu(kc), gpu(vc)
        mats.append(mt), gains.append(g), caches0.append((kc, vc)), gpu_layers.append(lw)
    spec = bl.BlockSpec(bl.BLOCK_DECODER_CACHED, hdim, inter, gpu_layers, nh, nkv, hd, EPS, slot=gpu(slot),
                        pos=gpu(pos), rope_table=bl.rope_table(theta, hd, 4096, DEV))
    tr = _trace(layers, m, hdim, inter, Q)
    tr["attn"] = torch.zeros((layers, m, hdim), dtype=torch.float32, device=DEV)
    y = bl.block_forward(spec, gpu(x), trace=tr)
    g_ = {k: host(v) for k, v in tr.items()}
    xin = x
    for l in range(layers):
        w = _oracle_weights(mats[l], gains[l])
        gl = gains[l] or {}
        s_qkv = oracle.forward(xin, w["qkv"], w["g_qkv"], [hdim, hdim + kvd, Q], gl.get("n_in"), EPS)
        assert_equal(g_["codes_in"][l], s_qkv["q"], f"layer {l} input codes")
        assert_equal(g_["acc_qkv"][l], s_qkv["acc"], f"layer {l} qkv acc")
        assert_equal(g_["qkv"][l], s_qkv["y"], f"layer {l} qkv")
        # RoPE on q and k, the appended cache rows
        qk = oracle.rope(g_["qkv"][l][:, :hdim + kvd], pos, nh + nkv, hd, theta)
        kc_gpu = host(gpu_layers[l].k_cache).view(np.uint16)
        vc_gpu = host(gpu_layers[l].v_cache).view(np.uint16)
        kc_ref, vc_ref = caches0[l][0].copy(), caches0[l][1].copy()
        oracle.kv_append(kc_ref, vc_ref, qk[:, hdim:], g_["qkv"][l][:, hdim + kvd:], slot, pos, nkv, hd)
        assert_equal(vc_gpu, vc_ref, f"layer {l} value cache")
        assert_equal(kc_gpu, kc_ref, f"layer {l} key cache")
        # attention over the GPU's caches
        att, vmag, smag, bad = oracle.attention(qk[:, :hdim], kc_gpu, vc_gpu, slot, pos, nh, nkv, hd)
        assert bad == 0
        assert _attn_bound_ok(g_["attn"][l], att, vmag, smag, hd, tmax).all(), f"layer {l} attention"
        # attn_sub_norm -> o_proj; h = x + o
        s_o = oracle.forward(g_["attn"][l], w["o"], [w["g_o"]], None, gl.get("n_attn"), EPS)
        assert_equal(g_["codes_attn"][l], s_o["q"], f"layer {l} attn_sub_norm codes")
        assert_equal(g_["acc_o"][l], s_o["acc"], f"layer {l} o acc")
        h = (xin.astype(np.float32) + s_o["y"]).astype(np.float32)
        assert_equal(g_["h"][l], h, f"layer {l} h")
        # MLP
        s_gu = oracle.forward(h, w["gu"], w["g_gu"], [inter, 2 * inter], gl.get("n_post"), EPS)
        assert_equal(g_["codes_post"][l], s_gu["q"], f"layer {l} post-norm codes")
        assert_equal(g_["acc_gate_up"][l], s_gu["acc"], f"layer {l} gate|up acc")
        assert_equal(g_["gate_up"][l], s_gu["y"], f"layer {l} gate|up")
        s_d = oracle.forward(oracle.relu2_mul(s_gu["y"], inter), w["down"], [w["g_down"]], None, gl.get("n_ffn"),
                             EPS)
        assert_equal(g_["codes_ffn"][l], s_d["q"], f"layer {l} ffn_sub_norm codes")
        assert_equal(g_["acc_down"][l], s_d["acc"], f"layer {l} down acc")
        x_next = (h + s_d["y"]).astype(np.float32)
        assert_equal(g_["x_out"][l], x_next, f"layer {l} output")
        xin = g_["x_out"][l]
    assert_equal(host(y), g_["x_out"][-1], "block output")
