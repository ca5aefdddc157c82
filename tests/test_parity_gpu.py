"""GPU (gfx950) against the CPU oracle, through the C ABI, element by element.

Bar: int8 activation codes, ternary codes / packed bytes (GPU given the
oracle's fp64 gamma) and int32 accumulators bit-exact; fp32 outputs and deq
within 1e-5 max relative error; the GPU's own gamma within 1e-6 relative.
Full-size workloads compare every code and sampled rows / columns of the
contraction, which the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_bitlinear_w1_amd import bitlinear as bl
from ternary_weight_bitlinear_w1_amd import synth

from _cases import (EPS, GAMMA_TOL, Matrix, assert_equal, assert_rel, note, seed, stacked)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_pack(mats):
    """Pack matrices on the GPU with the oracle's gamma, stacked along N."""
    parts = []
    for m in mats:
        p, g = bl.quantize_weights(gpu(m.w), gamma_in=gpu(np.array([m.gamma])))
        parts.append(p)
    return torch.cat(parts) if len(parts) > 1 else parts[0]


# ------------------------------------------------------------------------------ weights
@pytest.mark.parametrize("n,k", [(512, 256), (1, 16), (3, 48), (17, 272), (640, 2560), (2560, 6912)])
def test_quantize_weights(n, k):
    note(f"quantize_weights n={n} k={k}")
    m = Matrix(n, k, seed(1, n, k))
    packed, gamma = bl.quantize_weights(gpu(m.w))
    g = float(host(gamma)[0])
    assert abs(g - m.gamma) <= GAMMA_TOL * m.gamma
    packed_o, gamma_o = bl.quantize_weights(gpu(m.w), gamma_in=gpu(np.array([m.gamma])))
    assert float(host(gamma_o)[0]) == m.gamma
    assert_equal(host(packed_o), oracle.pack(m.codes), "packed bytes")
    # with its own gamma a code may differ only within |dgamma| / 2 of the threshold
    own, bad = oracle.unpack(host(packed), k)
    assert bad == 0
    flip = own != m.codes
    if flip.any():
        dist = np.abs(np.abs(m.w[flip].astype(np.float64)) - m.gamma / 2)
        assert np.all(dist <= abs(g - m.gamma) / 2 + 1e-300)
    assert bl.validate_packed(packed_o, k) == 0


def test_quantize_weights_deterministic_and_special():
    note("quantize_weights determinism, zero matrix, constant magnitude")
    m = Matrix(6912, 2560, seed(1, 99, 1))
    w = gpu(m.w)
    g1 = host(bl.quantize_weights(w)[1])
    g2 = host(bl.quantize_weights(w)[1])
    assert g1.tobytes() == g2.tobytes()
    z = np.zeros((32, 64), dtype=np.float32)
    p, g = bl.quantize_weights(gpu(z))
    assert host(g)[0] == 0.0
    assert_equal(host(p), oracle.pack(np.zeros((32, 64), np.int8)))
    c = (np.where(np.arange(32 * 64).reshape(32, 64) % 3 == 0, -1, 1) * np.float32(0.75)).astype(np.float32)
    p, g = bl.quantize_weights(gpu(c))
    assert host(g)[0] == 0.75
    assert_equal(host(p), oracle.pack(np.sign(c).astype(np.int8)))


def test_validate_packed_counts_invalid_fields():
    note("validate_packed on random bytes")
    rng = np.random.default_rng(3)
    p = rng.integers(0, 256, size=(37, 16), dtype=np.uint8)
    _, bad = oracle.unpack(p, 64)
    assert bl.validate_packed(gpu(p), 64) == bad


# ------------------------------------------------------------------------------ activations
# (17 to 128 rows take 1024-thread workgroups; (100, 9216) gives them 3 float4 per thread)
ACT_CASES = [(128, 256, 4), (1, 2560, 26), (4, 2560, 26), (16, 6912, 69), (130, 48, 0), (3, 16, 0),
             (5, 9216, 3), (1024, 512, 0), (64, 2560, 0), (17, 6912, 69), (100, 9216, 3), (1025, 2560, 26)]


def _edge_rows(x):
    x = x.copy()
    if x.shape[0] > 3:
        x[1] = 0.0
        x[2] = (x[2].astype(np.float64) * 2.0 ** -135).astype(np.float32)  # subnormal, 127 / a overflows
        x[3] = (x[3].astype(np.float64) * 1e30).astype(np.float32)
    if x.shape[0] > 5:
        x[4] = 0.0
        x[4, x.shape[1] // 2] = -3.5
        x[5] = (x[5].astype(np.float64) * 2.0 ** -70).astype(np.float32)
    return x


@pytest.mark.parametrize("m,k,nout", ACT_CASES)
def test_quantize_acts_absmax(m, k, nout):
    note(f"quantize_acts absmax m={m} k={k}")
    x = _edge_rows(synth.activations(seed(2, m, k), m, k, nout))
    codes, deq, rowsum = bl.quantize_acts(gpu(x))
    qo, do = oracle.quant_absmax(x)
    assert_equal(host(codes), qo, "codes")
    assert_equal(host(deq), do, "deq")
    assert_equal(host(rowsum), qo.astype(np.int64).sum(axis=1).astype(np.int32), "row sums")


@pytest.mark.parametrize("m,k,with_gain", [(128, 256, False), (16, 2560, True), (7, 6912, False), (64, 2560, True),
                                           (3, 9216, True), (1500, 1024, True)])
def test_quantize_acts_rmsnorm(m, k, with_gain):
    note(f"quantize_acts rmsnorm m={m} k={k} gain={with_gain}")
    x = _edge_rows(synth.activations(seed(3, m, k), m, k, 2))
    gain = (1.0 + 0.2 * synth.normal_f32(seed(3, m, 99), k)).astype(np.float32) if with_gain else None
    codes, deq, rowsum = bl.quantize_acts(gpu(x), bl.ACT_RMSNORM, None if gain is None else gpu(gain), EPS)
    qo, do = oracle.quant_rms(x, gain, EPS)
    assert_equal(host(codes), qo, "codes")
    assert_rel(host(deq), do, what="deq")
    assert_equal(host(rowsum), qo.astype(np.int64).sum(axis=1).astype(np.int32), "row sums")


@pytest.mark.parametrize("m,inter,with_gain", [(1024, 2048, False), (1, 6912, False), (16, 6912, True), (5, 48, True),
                                               (40, 6912, True)])
def test_quantize_acts_relu2(m, inter, with_gain):
    note(f"quantize_acts relu2 m={m} I={inter}")
    gu = synth.activations(seed(4, m, inter), m, 2 * inter)
    gu[0, :7] = -0.0
    gain = (1.0 + 0.2 * synth.normal_f32(seed(4, m, 98), inter)).astype(np.float32) if with_gain else None
    codes, deq, _ = bl.quantize_acts(gpu(gu), bl.ACT_RELU2_RMSNORM, None if gain is None else gpu(gain), EPS)
    mi = oracle.relu2_mul(gu, inter)
    qo, do = oracle.quant_rms(mi, gain, EPS)
    assert_equal(host(codes), qo, "codes")
    assert_rel(host(deq), do, what="deq")
    assert np.all(host(codes)[gu[:, :inter] <= 0] == 0)


# ------------------------------------------------------------------------------ forward
def _check_forward(x, mats, path, what):
    codes, gammas, ends = stacked(mats)
    packed = gpu_pack(mats)
    k = x.shape[1]
    y, acc = bl.forward(packed, k, [float(np.float32(g)) for g in gammas], ends, x=gpu(x), want_acc=True, path=path)
    ref = oracle.forward(x, codes, gammas, ends)
    assert_equal(host(acc), ref["acc"], f"{what} acc")
    assert_rel(host(y), ref["y"], what=f"{what} y")
    assert_equal(host(y), ref["y"], f"{what} y bit-exact")
    return y


def test_forward_single_layer():
    """K=256 -> N=512, M=128 tokens, 4 outlier channels."""
    note("forward single layer 128x256x512")
    x = synth.activations(seed(1, 0, 2), 128, 256, 4)
    _check_forward(x, [Matrix(512, 256, seed(1, 0, 1))], bl.PATH_PREFILL, "single layer")


RAGGED = [(1, 40, 48), (3, 200, 80), (17, 130, 272), (130, 1000, 64), (64, 96, 16), (257, 129, 2576),
          (16, 16, 16), (2, 33, 4112), (300, 700, 1040),
          # shapes the pipelined kernel takes (N % 128 == 0, K % 128 == 0): K-chunk counts 1, 2, 3,
          # 5, 9 and M not a multiple of the tile; past 64 tokens, where 128-row tiles would leave
          # half of the CUs idle, the 64 x 64 tile
          (130, 512, 256), (65, 384, 384), (40, 768, 640), (333, 1280, 1152), (20, 256, 128), (257, 2560, 2560),
          # enough 128-row tiles: 128 x 256 and 128 x 128
          (1100, 4096, 384), (2000, 1152, 256),
          # few-token shapes of the dot-product decode kernel (one token, K % 64 == 0) and of the
          # MFMA decode kernel (2 to 4 tokens): rows not a multiple of 8, K from one partial line
          # to 8192, every split of K over waves
          (1, 77, 64), (2, 200, 320), (3, 1000, 576), (4, 40, 8192), (1, 9000, 1024), (4, 5000, 448),
          # 5..16 tokens over at least 8192 rows: two row tiles per workgroup, ragged rows and K
          (12, 8200, 320), (6, 8224, 2576),
          # 5..16 tokens over at least 12800 rows and at most 16 supersteps of 256 k: four row tiles
          # per workgroup, one wave per superstep (4 to 16 waves, some without a superstep), ragged
          (16, 13824, 2560), (9, 12864, 4096), (12, 12848, 1040), (13, 12800, 1536), (10, 12816, 208),
          (16, 12816, 2832), (5, 12864, 2560), (8, 12816, 1040),
          # long rows: one token past the dot-product kernel's 8192 (sixteen waves of four supersteps,
          # per-lane code loads), and past 16 waves x 4 supersteps (the looping kernel)
          (1, 70, 8256), (3, 100, 16400),
          # few output tiles, where K is split into ranges (16, 8, 4 here) whose int32 partial sums a
          # second kernel adds, and neighbours that are not split
          (9, 512, 4096), (5, 256, 2048), (48, 1024, 3072), (37, 512, 1024), (100, 384, 768),
          # 17..64 tokens with K % 256 == 0 (AUTO takes the skinny kernel): one and two token tiles,
          # ragged rows, few and many supersteps per wave
          (17, 130, 512), (32, 1000, 768), (33, 48, 2560), (64, 2600, 6912), (50, 3000, 1024),
          # at most 64 tokens, one work item per CU and an even chunk count: two K groups per
          # workgroup (200 tiles unsplit; 24 tiles split in two; exactly 256 items, unsplit and
          # split four ways)
          (61, 12800, 512), (50, 1536, 1024), (64, 16384, 256), (47, 4096, 2048),
          # the 8-wave 128 x 320 tile (N % 320 == 0 and at least one tile per CU): ragged last row
          # tile; two rounds of tiles with one K chunk each
          (4000, 2560, 256), (4096, 5120, 128),
          # 576 tiles of 128 x 256 for 512 workgroups: a second, nearly empty round
          (4000, 4608, 128)]


@pytest.mark.parametrize("m,n,k", RAGGED)
def test_forward_ragged(m, n, k):
    note(f"forward ragged m={m} n={n} k={k}")
    x = _edge_rows(synth.activations(seed(5, m, k), m, k, 1 if k >= 100 else 0))
    n1 = n // 3 + 1 if n % 128 else n // 2
    mats = [Matrix(n1, k, seed(5, n, 1)), Matrix(n - n1, k, seed(5, n, 2), sigma=0.05)]
    paths = [bl.PATH_PREFILL, bl.PATH_AUTO] + ([bl.PATH_DECODE] if m <= 16 else [])
    ys = [host(_check_forward(x, mats, p, f"path {p}")) for p in paths]
    for y in ys[1:]:
        assert_equal(y, ys[0], "decode == prefill")


# ------------------------------------------------------------------------------ gated up-projection
GLU = [(200, 512, 1024), (130, 384, 256), (65, 256, 2560), (257, 640, 640),  # gating fused, 64 x 128 tiles
       (1000, 8448, 128),  # 528 tiles of 128 x 256 for 512 workgroups
       (1100, 2048, 256),  # 144 tiles of 128 x 256
       (300, 200, 1040), (40, 256, 512), (5, 512, 512), (1, 96, 320)]          # gate|up through the workspace


@pytest.mark.parametrize("m,inter,k", GLU)
def test_forward_relu2_glu(m, inter, k):
    """fl32(max(g, 0)^2 * u) of the gate|up projection, against the oracle's
    O6 of its O8 output, bit for bit, and equal to forward + gating on the GPU."""
    note(f"forward relu2 glu m={m} inter={inter} k={k}")
    x = synth.activations(seed(8, m, k), m, k, 1 if k >= 100 else 0)
    mats = [Matrix(inter, k, seed(8, inter, 1)), Matrix(inter, k, seed(8, inter, 2), sigma=0.05)]
    codes, gammas, ends = stacked(mats)
    packed = gpu_pack(mats)
    g = [float(np.float32(v)) for v in gammas]
    ref = oracle.relu2_mul(oracle.forward(x, codes, gammas, ends)["y"], inter)
    for path in [bl.PATH_AUTO, bl.PATH_PREFILL] + ([bl.PATH_DECODE] if m <= 16 else []):
        y = host(bl.forward_relu2_glu(packed, k, g, x=gpu(x), path=path))
        assert_equal(y, ref, f"gated y path {path}")
    gu = bl.forward(packed, k, g, ends, x=gpu(x), path=bl.PATH_PREFILL)
    assert_equal(host(bl.forward_relu2_glu(packed, k, g, x=gpu(x))), oracle.relu2_mul(host(gu), inter),
                 "gated == forward + gating")


def test_forward_relu2_glu_full_size():
    """M=4096 gate|up 2560 -> 2 x 6912 with the gating fused: sampled rows against
    the oracle (tokens are independent), and determinism."""
    note("forward relu2 glu m=4096")
    m, k, inter = 4096, 2560, 6912
    mats = [Matrix(inter, k, seed(4, 0, 1)), Matrix(inter, k, seed(4, 0, 2))]
    codes, gammas, ends = stacked(mats)
    packed = gpu_pack(mats)
    g = [float(np.float32(v)) for v in gammas]
    x = synth.activations(seed(4, 1, 7), m, k)
    y = host(bl.forward_relu2_glu(packed, k, g, x=gpu(x)))
    rows = np.array([0, 1, 127, 128, 2047, 4095])
    ref = oracle.relu2_mul(oracle.forward(x[rows], codes, gammas, ends)["y"], inter)
    assert_equal(y[rows], ref, "sampled rows")
    assert_equal(host(bl.forward_relu2_glu(packed, k, g, x=gpu(x))), y, "determinism")


# ------------------------------------------------------------------------------ online mode
ONLINE = [(1, [512], 256), (37, [100, 300], 512), (4, [6912, 13824], 2560), (130, [2560], 6912), (0, [64], 128)]


@pytest.mark.parametrize("m,seg,k", ONLINE)
def test_forward_online(m, seg, k):
    """Ternarize fp32 masters inside the forward: gamma per segment within 1e-6 of
    the oracle's; y and acc bit-exact against the oracle run with the GPU's gamma
    (a code can only differ within |dgamma| / 2 of its threshold); equal to
    quantize_weights + forward on the GPU."""
    note(f"forward online m={m} seg={seg} k={k}")
    n = seg[-1]
    lo = [0] + seg[:-1]
    mats = [Matrix(hi - a, k, seed(9, n + j, k), sigma=0.02 + 0.01 * j) for j, (a, hi) in enumerate(zip(lo, seg))]
    w = np.concatenate([mt.w for mt in mats])
    x = synth.activations(seed(9, m, k), max(m, 1), k, 1 if k >= 100 else 0)[:m]
    y, acc, gamma = bl.forward_online(gpu(w), seg, x=gpu(x), want_acc=True)
    g = host(gamma)
    for j, mt in enumerate(mats):
        assert abs(g[j] - mt.gamma) <= GAMMA_TOL * mt.gamma, (j, g[j], mt.gamma)
    codes = np.concatenate([oracle.ternarize(mt.w, float(g[j])) for j, mt in enumerate(mats)])
    if m == 0:
        assert y.shape == (0, n)
        return
    ref = oracle.forward(x, codes, [float(v) for v in g], seg)
    assert_equal(host(acc), ref["acc"], "online acc")
    assert_equal(host(y), ref["y"], "online y")
    packed = torch.cat([bl.quantize_weights(gpu(mt.w))[0] for mt in mats])
    y_p = bl.forward(packed, k, [float(np.float32(v)) for v in g], seg, x=gpu(x))
    assert_equal(host(y_p), host(y), "online == quantize_weights + forward")


@pytest.mark.parametrize("m,seg,k", [(1, [6912, 13824], 2560), (37, [100, 300], 512), (130, [2560], 6912)])
def test_forward_online_bf16(m, seg, k):
    """bfloat16 masters ("The two checkpoints": the bf16 checkpoint), read as their
    exact fp32 values: gamma per segment against the oracle's absmean of the
    widened masters (within 1e-6), y and acc bit-exact against the oracle run with
    the GPU's gamma, and equal to the fp32-master call on the widened values."""
    note(f"forward online bf16 m={m} seg={seg} k={k}")
    n = seg[-1]
    lo = [0] + seg[:-1]
    bits = np.concatenate([oracle.round_bf16(synth.weights(seed(10, n + j, k), hi - a, k, 0.02 + 0.01 * j))
                           for j, (a, hi) in enumerate(zip(lo, seg))])
    wide = oracle.bf16_to_f32(bits)
    x = synth.activations(seed(10, m, k), m, k, 1)
    y, acc, gamma = bl.forward_online(gpu(bits), seg, x=gpu(x), want_acc=True)
    g = host(gamma)
    for j, (a, hi) in enumerate(zip(lo, seg)):
        go = oracle.absmean(wide[a:hi])
        assert abs(g[j] - go) <= GAMMA_TOL * go, (j, g[j], go)
    codes = np.concatenate([oracle.ternarize(wide[a:hi], float(g[j])) for j, (a, hi) in enumerate(zip(lo, seg))])
    ref = oracle.forward(x, codes, [float(v) for v in g], seg)
    assert_equal(host(acc), ref["acc"], "online bf16 acc")
    assert_equal(host(y), ref["y"], "online bf16 y")
    y32, g32 = bl.forward_online(gpu(wide), seg, x=gpu(x))
    assert_equal(host(g32), g, "gamma from the widened fp32 masters")
    assert_equal(host(y32), host(y), "bf16 masters == their fp32 widening")


# one token: the contraction that forms the codes from the masters as it reads
# them (fp32 up to k = 4096, bfloat16 up to 8192), with a partial last line
# (k = 2576) and segments of ragged length; fp32 at k = 6912 takes the packed
# path instead
ONLINE_ONE = [("f32", [512], 256), ("f32", [100, 257], 2576), ("bf16", [6912, 13824], 2560),
              ("bf16", [300, 301, 700], 6912), ("bf16", [37], 8192), ("f32", [64, 200], 6912)]


@pytest.mark.parametrize("dt,seg,k", ONLINE_ONE)
def test_forward_online_one_token(dt, seg, k):
    """One token in the online mode: y and acc bit-exact against the oracle run
    with the GPU's gammas, the gammas within 1e-6 of the oracle's, and y, acc and
    gammas equal to the packed path (path PREFILL, which ternarizes into the
    workspace first), also when the token's codes are given."""
    note(f"forward online one token {dt} seg={seg} k={k}")
    n = seg[-1]
    lo = [0] + seg[:-1]
    w = np.concatenate([synth.weights(seed(11, n + j, k), hi - a, k, 0.02 + 0.01 * j)
                        for j, (a, hi) in enumerate(zip(lo, seg))])
    if dt == "bf16":
        bits = oracle.round_bf16(w)
        wide, wt = oracle.bf16_to_f32(bits), gpu(bits)
    else:
        wide, wt = w, gpu(w)
    x = synth.activations(seed(11, 1, k), 1, k, 1)
    y, acc, gamma = bl.forward_online(wt, seg, x=gpu(x), want_acc=True)
    g = host(gamma)
    for j, (a, hi) in enumerate(zip(lo, seg)):
        go = oracle.absmean(wide[a:hi])
        assert abs(g[j] - go) <= GAMMA_TOL * go, (j, g[j], go)
    codes = np.concatenate([oracle.ternarize(wide[a:hi], float(g[j])) for j, (a, hi) in enumerate(zip(lo, seg))])
    ref = oracle.forward(x, codes, [float(v) for v in g], seg)
    assert_equal(host(acc), ref["acc"], "online one-token acc")
    assert_equal(host(y), ref["y"], "online one-token y")
    y_p, acc_p, g_p = bl.forward_online(wt, seg, x=gpu(x), want_acc=True, path=bl.PATH_PREFILL)
    assert_equal(host(g_p), g, "gammas of the packed path")
    assert_equal(host(acc_p), host(acc), "acc of the packed path")
    assert_equal(host(y_p), host(y), "y of the packed path")
    c, d, r = bl.quantize_acts(gpu(x))
    y_c, g_c = bl.forward_online(wt, seg, codes=c, deq=d, rowsum=r)
    assert_equal(host(y_c), host(y), "codes given")
    y_c2, _ = bl.forward_online(wt, seg, codes=c, deq=d)
    assert_equal(host(y_c2), host(y), "codes given, row sum formed")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("special", [np.inf, np.nan])
def test_forward_online_one_token_special_masters(dt, special):
    """A segment whose masters hold an infinity or a NaN: its gamma is inf or NaN,
    no weight passes the threshold test (as in the oracle's fp64 test), and its
    outputs are NaN; the other segment is untouched (bit-exact against the
    oracle), and the one-token path equals the packed path."""
    note(f"forward online one token, {dt} masters with {special}")
    k, seg = 512, [64, 136]
    w = np.concatenate([synth.weights(seed(12, 1, k), 64, k, 0.02), synth.weights(seed(12, 2, k), 72, k, 0.03)])
    w[100, 7] = special
    if dt == "bf16":
        bits = oracle.round_bf16(w)
        wide, wt = oracle.bf16_to_f32(bits), gpu(bits)
    else:
        wide, wt = w, gpu(w)
    x = synth.activations(seed(12, 1, k), 1, k, 1)
    y, acc, gamma = bl.forward_online(wt, seg, x=gpu(x), want_acc=True)
    g = host(gamma)
    assert abs(g[0] - oracle.absmean(wide[:64])) <= GAMMA_TOL * g[0]
    assert (np.isinf(g[1]) if special == np.inf else np.isnan(g[1])), g[1]
    codes0 = oracle.ternarize(wide[:64], float(g[0]))
    ref = oracle.forward(x, codes0, [float(g[0])], [64])
    assert_equal(host(acc)[:, :64], ref["acc"], "finite segment acc")
    assert_equal(host(y)[:, :64], ref["y"], "finite segment y")
    assert_equal(host(acc)[:, 64:], np.zeros((1, 72), np.int32), "no weight passes the test")
    assert np.isnan(host(y)[:, 64:]).all()
    y_p, acc_p, g_p = bl.forward_online(wt, seg, x=gpu(x), want_acc=True, path=bl.PATH_PREFILL)
    assert_equal(host(acc_p), host(acc), "acc of the packed path")
    assert_equal(host(y_p)[:, :64], host(y)[:, :64], "y of the packed path")
    assert np.isnan(host(y_p)[:, 64:]).all()


def test_forward_codes_in_path():
    note("forward with pre-quantized codes")
    m, k, n = 37, 512, 300
    x = synth.activations(seed(6, m, k), m, k, 5)
    mat = Matrix(n, k, seed(6, 0, 1))
    packed = gpu_pack([mat])
    codes, deq, rowsum = bl.quantize_acts(gpu(x))
    g = [mat.gamma_f]
    y_x = host(bl.forward(packed, k, g, x=gpu(x)))
    y_c = host(bl.forward(packed, k, g, codes=codes, deq=deq))
    y_r = host(bl.forward(packed, k, g, codes=codes, deq=deq, rowsum=rowsum))
    assert_equal(y_c, y_x)
    assert_equal(y_r, y_x)


@pytest.mark.parametrize("m", [1, 4, 16, 64])
@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_forward_decode_full_size(m, proj):
    """Decode sweep at the 2B4T projection shapes, gate|up with one gamma each; the
    prefill kernel at these few-tile shapes splits K (and m = 64 takes only it)."""
    note(f"forward decode {proj} m={m}")
    if proj == "gate_up":
        k = 2560
        mats = [Matrix(6912, k, seed(3, 0, 1)), Matrix(6912, k, seed(3, 0, 2))]
    else:
        k = 6912
        mats = [Matrix(2560, k, seed(3, 0, 3))]
    x = synth.activations(seed(3, m, k), m, k, synth.outlier_count(k))
    y_pre = _check_forward(x, mats, bl.PATH_PREFILL, f"prefill {proj}")
    y_auto = _check_forward(x, mats, bl.PATH_AUTO, f"auto {proj}")  # m = 64: the skinny kernel
    assert_equal(host(y_auto), host(y_pre), "auto == prefill")
    if m <= 16:
        y_dec = _check_forward(x, mats, bl.PATH_DECODE, f"decode {proj}")
        assert_equal(host(y_dec), host(y_pre), "decode == prefill")


@pytest.mark.parametrize("m", [1, 4, 16])
@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_forward_decode_tall(m, proj):
    """The decode kernels in one launch over many stacked copies of a 2B4T matrix
    (the form the benchmark streams 628 MB with): 16 copies, 110,592 gate rows or
    40,960 down rows. One copy is checked against the oracle (codes, int32 sums
    and outputs); every copy of the tall launch must equal it bit for bit."""
    note(f"forward decode tall {proj} m={m}")
    k, n = (2560, 6912) if proj == "gate_up" else (6912, 2560)
    mat = Matrix(n, k, seed(5, 0, 1 if proj == "gate_up" else 2))
    x = synth.activations(seed(5, m, k), m, k, synth.outlier_count(k))
    y_one = host(_check_forward(x, [mat], bl.PATH_DECODE, f"decode {proj}"))
    copies = 16
    tall = gpu_pack([mat]).repeat(copies, 1)
    y_tall, acc_tall = bl.forward(tall, k, [mat.gamma_f], [copies * n], x=gpu(x), want_acc=True,
                                  path=bl.PATH_DECODE)
    yt, at = host(y_tall), host(acc_tall)
    ref_acc = oracle.forward(x, mat.codes, [mat.gamma], [n])["acc"]
    for c in range(copies):
        assert_equal(yt[:, c * n:(c + 1) * n], y_one, f"copy {c} outputs")
        assert_equal(at[:, c * n:(c + 1) * n], ref_acc, f"copy {c} int32 sums")


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_forward_prefill_full_size(proj):
    """M=4096 prefill at the 2B4T shapes: every code, sampled rows and columns of the
    contraction, and determinism."""
    note(f"forward prefill {proj} m=4096")
    if proj == "gate_up":
        k, mats = 2560, [Matrix(6912, 2560, seed(4, 0, 1)), Matrix(6912, 2560, seed(4, 0, 2))]
    else:
        k, mats = 6912, [Matrix(2560, 6912, seed(4, 0, 3))]
    m = 4096
    x = synth.activations(seed(4, 1 if proj == "gate_up" else 2, 7), m, k)
    codes_o, gammas, ends = stacked(mats)
    packed = gpu_pack(mats)
    n = packed.shape[0]
    gf = [float(np.float32(g)) for g in gammas]
    xg = gpu(x)
    codes, deq, rowsum = bl.quantize_acts(xg)
    qo, do = oracle.quant_absmax(x)
    assert_equal(host(codes), qo, "codes (all rows)")
    assert_equal(host(deq), do, "deq (all rows)")
    y, acc = bl.forward(packed, k, gf, ends, x=xg, want_acc=True, path=bl.PATH_PREFILL)
    y2 = bl.forward(packed, k, gf, ends, x=xg, path=bl.PATH_PREFILL)
    yh, acch = host(y), host(acc)
    assert yh.tobytes() == host(y2).tobytes()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 2047, 4095], rng.integers(0, m, 4)]))
    ref = oracle.forward(x[rows], codes_o, gammas, ends)
    assert_equal(acch[rows], ref["acc"], "acc (sampled rows)")
    assert_equal(yh[rows], ref["y"], "y (sampled rows)")
    cols = np.unique(np.concatenate([[0, n - 1, ends[0] - 1, ends[0] % n], rng.integers(0, n, 4)]))
    acc_c = oracle.contract(qo, codes_o[cols])
    assert_equal(acch[:, cols], acc_c, "acc (sampled columns, all rows)")
    for j, c in enumerate(cols):
        seg = int(np.searchsorted(ends, c, side="right"))
        y_col = oracle.rescale(acc_c[:, j:j + 1], do, [gammas[seg]], [1])
        assert_equal(yh[:, c:c + 1], y_col, f"y (column {c}, all rows)")


def test_forward_codes_past_32bit_offsets():
    """Codes of 65600 x 65536 bytes (4.3 GB, past 2^32): rows whose byte offset
    does not fit 32 bits contract like the first ones. Sampled rows on both sides
    of 2^31 and 2^32 are checked against the oracle: int32 sums and fp32 outputs
    bit for bit."""
    m, n, k = 65600, 256, 65536
    note(f"forward past 32-bit offsets m={m} n={n} k={k}")
    mat = Matrix(n, k, seed(7, 1, 1))
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed(7, 1, 2))
    codes = torch.randint(-127, 128, (m, k), dtype=torch.int8, device=DEV, generator=gen)
    deq = (torch.rand((m,), dtype=torch.float32, device=DEV, generator=gen) + 0.5) / 127.0
    y, acc = bl.forward(gpu(oracle.pack(mat.codes)), k, [mat.gamma_f], codes=codes, deq=deq, want_acc=True,
                        path=bl.PATH_PREFILL)
    rows = [0, 1, 32767, 32768, 65535, 65536, 65599]
    idx = torch.tensor(rows, device=DEV)
    q = host(codes.index_select(0, idx))
    d = host(deq.index_select(0, idx))
    a_gpu, y_gpu = host(acc.index_select(0, idx)), host(y.index_select(0, idx))
    del codes, y, acc
    acc_o = oracle.contract(q, mat.codes)
    assert_equal(a_gpu, acc_o, "acc")
    assert_equal(y_gpu, oracle.rescale(acc_o, d, [mat.gamma], [n]), "y")


# ------------------------------------------------------------------------------ empty token batches
def test_empty_token_batches():
    """m = 0 is a no-op on every per-token entry point: each returns success with
    an empty output, and the decode, prefill and automatic paths agree on it."""
    note("empty token batches")
    k, n, inter = 256, 96, 128
    mat = Matrix(n, k, seed(8, 0, 1))
    packed = gpu(oracle.pack(mat.codes))
    g = [mat.gamma_f]
    x0 = torch.empty((0, k), dtype=torch.float32, device=DEV)
    for mode in (bl.ACT_ABSMAX, bl.ACT_RMSNORM):
        codes, deq, rowsum = bl.quantize_acts(x0, mode)
        assert tuple(codes.shape) == (0, k) and deq.numel() == 0 and rowsum.numel() == 0
    codes, deq, rowsum = bl.quantize_acts(torch.empty((0, 2 * k), device=DEV), bl.ACT_RELU2_RMSNORM)
    assert tuple(codes.shape) == (0, k)
    for path in (bl.PATH_AUTO, bl.PATH_PREFILL, bl.PATH_DECODE):
        y, acc = bl.forward(packed, k, g, x=x0, want_acc=True, path=path)
        assert tuple(y.shape) == (0, n) and tuple(acc.shape) == (0, n)
        y = bl.forward(packed, k, g, codes=torch.empty((0, k), dtype=torch.int8, device=DEV),
                       deq=torch.empty(0, device=DEV), path=path)
        assert tuple(y.shape) == (0, n)
    gu = Matrix(2 * inter, k, seed(8, 0, 2))
    y = bl.forward_relu2_glu(gpu(oracle.pack(gu.codes)), k, [gu.gamma_f, gu.gamma_f], x=x0)
    assert tuple(y.shape) == (0, inter)
    head = torch.zeros((64, k), dtype=torch.uint16, device=DEV)
    assert tuple(bl.lm_head(x0, head).shape) == (0, 64)
    assert tuple(bl.embed(torch.empty(0, dtype=torch.int64, device=DEV), head).shape) == (0, k)
    pos = torch.empty(0, dtype=torch.int64, device=DEV)
    bl.rope(torch.empty((0, 256), device=DEV), pos, 2, 128, bl.rope_table(5e5, 128, 16, DEV))
    kc = torch.zeros((1, 1, 16, 128), dtype=torch.uint16, device=DEV)
    vc = torch.zeros_like(kc)
    o = bl.attention_decode(torch.empty((0, 256), device=DEV), kc, vc, pos, pos, 2)
    assert tuple(o.shape) == (0, 256)
    assert not kc.view(torch.int16).any() and not vc.view(torch.int16).any()
