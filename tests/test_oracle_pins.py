"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it checks. None of them re-types the oracle's own
formula: they use hand-derived fixtures (tests/golden), exact rational
arithmetic, closed forms, invariants, brute force on tiny inputs, library
routines on special cases, and an independent fp64 formulation of the block
written from the block equations.

Pages: [card] = "BitNet b1.58 2B4T - Scaling Native 1-bit LLM" model card;
[nnterp] = "nnterp encyclopedia: BitNet b1.58".
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from ternary_weight_bitlinear_w1_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F32_ULP = 2.0 ** -23


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ O1 / O2
def test_golden_ternary_codes():
    """[nnterp] "The projections quantize their inputs and weights"; [card] "Model Details"."""
    for case in gold("ternary_codes.json")["cases"]:
        w = np.array([case["w"]], dtype=np.float32)
        g = oracle.absmean(w)
        assert g == case["gamma"]
        assert oracle.ternarize(w, g).tolist() == [case["codes"]]


@pytest.mark.parametrize("a", [0.75, 0.02, 1e-3, 3.0])
def test_P1_constant_magnitude_gives_exact_gamma(a):
    """mean|W| of a matrix whose entries all have magnitude a is a, exactly."""
    r = rng(1)
    a32 = np.float32(a)
    w = (np.where(r.random((37, 48)) < 0.5, -1, 1) * a32).astype(np.float32)
    assert oracle.absmean(w) == float(a32)
    c = oracle.ternarize(w, oracle.absmean(w))
    assert np.array_equal(c, np.sign(w).astype(np.int8))


def test_P1_grid_weights_exact_rational_mean():
    """W on a 2^-10 grid: the fp64 sum is exact, so gamma is the correctly rounded
    rational mean sum|W| / (N K)."""
    r = rng(2)
    wi = r.integers(-3000, 3001, size=(19, 33))
    w = (wi / 1024.0).astype(np.float32)
    exact = Fraction(int(np.abs(wi).sum()), 1024 * wi.size)
    assert oracle.absmean(w) == float(exact)


def test_P1_bf16_masters_exact_rational_mean():
    """[nnterp] "The two checkpoints": the bf16 checkpoint stores its weights in
    bfloat16 and ternarizes them in every forward. The oracle takes gamma over the
    exactly widened values: for bfloat16 weights of N(0, 0.02) (8 significant
    bits, exponents within a few dozen binades) the fp64 sum is exact, so gamma is
    the correctly rounded rational mean of the bfloat16 values themselves; a
    constant magnitude a gives gamma = a; codes split exactly at gamma / 2."""
    r = rng(3)
    bits = oracle.round_bf16((0.02 * r.normal(size=(23, 48))).astype(np.float32))
    wide = oracle.bf16_to_f32(bits)
    exact = sum((Fraction(float(v)).__abs__() for v in wide.reshape(-1)), Fraction(0)) / wide.size
    g = oracle.absmean(wide)
    assert g == float(exact)
    c = oracle.ternarize(wide, g)
    half = exact / 2
    want = np.array([0 if abs(Fraction(float(v))) <= half else (1 if v > 0 else -1) for v in wide.reshape(-1)])
    assert np.array_equal(c.reshape(-1), want)
    a_bits = 0x3C23  # bfloat16 of 0.00994873046875
    const = np.where(r.random((9, 32)) < 0.5, a_bits, a_bits | 0x8000).astype(np.uint16)
    assert oracle.absmean(oracle.bf16_to_f32(const)) == 0.00994873046875


def test_P2_codes_match_exact_rational_threshold():
    """Brute force: code = sign(W) * [ |W| > mean|W| / 2 ] in exact rationals
    (round(W / gamma) clipped to [-1, 1], ties to even)."""
    r = rng(3)
    for trial in range(20):
        n, k = r.integers(1, 9), r.integers(1, 17)
        w = (r.standard_normal((n, k)) * r.choice([0.02, 1.0, 50.0])).astype(np.float32)
        if trial % 4 == 0:  # quarter-grid values: exact ties with gamma / 2 become likely
            w = (r.integers(-8, 9, size=(n, k)) / 4.0).astype(np.float32)
        s = sum(Fraction(float(abs(v))) for v in w.ravel())
        half = s / (2 * w.size)
        want = np.array([[int(np.sign(v)) if Fraction(float(abs(v))) > half else 0 for v in row] for row in w])
        got = oracle.ternarize(w, oracle.absmean(w))
        assert set(np.unique(got)) <= {-1, 0, 1}
        bad = np.argwhere(got != want)
        for i, j in bad:  # only allowed within the fp64 rounding of gamma
            dist = abs(Fraction(float(abs(w[i, j]))) - half)
            assert dist <= half * Fraction(1, 2 ** 50), (trial, i, j)


def test_P2_tie_rounds_to_zero():
    """A weight exactly at gamma / 2 is a half-way case of round(W / gamma): it goes to 0."""
    w = np.array([[0.625, -0.625, 3.75, 0.0]], dtype=np.float32)  # sum 5, mean 1.25, half 0.625
    assert oracle.absmean(w) == 1.25
    assert oracle.ternarize(w, 1.25).tolist() == [[0, 0, 1, 0]]
    # one float step above the tie becomes +-1
    up = np.nextafter(np.float32(0.625), np.float32(1))
    assert oracle.ternarize(np.array([[up, -up]], dtype=np.float32), 1.25).tolist() == [[1, -1]]


def test_P3_small_weight_edit_is_reternarized_away():
    """[nnterp] "The projections quantize their inputs and weights": adding 0.1 * mean|W|
    to one weight leaves the ternarized weight unchanged (when that weight is not
    within 0.2 * mean|W| of the threshold)."""
    w = synth.weights(synth.stream_seed(7, tensor=synth.T_WEIGHT), 64, 256)
    g = oracle.absmean(w)
    c = oracle.ternarize(w, g)
    r = rng(4)
    checked = 0
    for idx in r.permutation(w.size)[:400]:
        i, j = divmod(int(idx), 256)
        v = float(w[i, j])
        if abs(abs(v) - g / 2) < 0.2 * g or abs(abs(v + 0.1 * g) - g / 2) < 0.1 * g:
            continue
        w2 = w.copy()
        w2[i, j] = np.float32(v + 0.1 * g)
        c2 = oracle.ternarize(w2, oracle.absmean(w2))
        assert np.array_equal(c, c2)
        checked += 1
    assert checked > 100


# ------------------------------------------------------------------ O3
def test_golden_pack_layout():
    """Four to a byte ([nnterp] "The two checkpoints"); bytes derived by hand from the layout rule."""
    for case in gold("pack_layout.json")["cases"]:
        c = np.array([case["codes"]], dtype=np.int8)
        p = oracle.pack(c)
        assert p.shape == (1, c.shape[1] // 4)
        assert p.ravel().tolist() == case["bytes"]
        back, bad = oracle.unpack(p, c.shape[1])
        assert bad == 0 and np.array_equal(back, c)


def test_P4_roundtrip_every_dword_pattern():
    """unpack(pack(c)) == c over all 3^16 patterns of one 16-code group, and
    pack(unpack(p)) == p for every valid packed dword (pack is a bijection)."""
    n = 3 ** 16
    idx = np.arange(n, dtype=np.int64)
    c = np.empty((n, 16), dtype=np.int8)
    for d in range(16):
        c[:, d] = (idx // (3 ** d)) % 3 - 1
    del idx
    p = oracle.pack(c)
    back, bad = oracle.unpack(p, 16)
    assert bad == 0
    assert np.array_equal(back, c)
    del back, c
    words = p.view(np.uint32).ravel()
    assert np.unique(words).size == n  # distinct codes give distinct words
    p2 = oracle.pack(oracle.unpack(p, 16)[0])
    assert np.array_equal(p2, p)


def test_P4_invalid_field_detected():
    """Field value 3 is not a ternary code: unpack counts it."""
    r = rng(5)
    p = r.integers(0, 256, size=(8, 16), dtype=np.uint8)
    fields = np.stack([(p >> s) & 3 for s in (0, 2, 4, 6)])
    _, bad = oracle.unpack(p, 64)
    assert bad == int((fields == 3).sum()) and bad > 0


# ------------------------------------------------------------------ five codes to a byte (R18)
def test_golden_base3_layout():
    """[tiny] "O que é", "Arquivos": a storage denser than two bits per weight; layout R18."""
    for case in gold("base3_layout.json")["cases"]:
        c = np.array([case["codes"]], dtype=np.int8)
        p = oracle.pack_base3(c)
        assert p.tolist() == [case["bytes"]]
        back, bad = oracle.unpack_base3(p, c.shape[1])
        assert bad == 0 and np.array_equal(back, c)


def test_base3_every_byte_value():
    """Each of the 243 valid bytes is five base-3 digits: decoding then encoding
    gives the byte back (a bijection between 3^5 code patterns and 0..242), and
    the digits are those of the integer division by 1, 3, 9, 27, 81."""
    v = np.arange(243)
    codes = np.stack([(v // 3 ** i) % 3 - 1 for i in range(5)], axis=1).astype(np.int8)  # [243][5]
    p = oracle.pack_base3(codes)
    assert np.array_equal(p[:, 0], v.astype(np.uint8))
    assert (p[:, 1:] == 121).all()
    back, bad = oracle.unpack_base3(p, 5)
    assert bad == 0 and np.array_equal(back, codes)


def test_base3_invalid_bytes_detected():
    """Bytes 243..255 are not five ternary digits: unpack counts them (only in
    bytes that hold codes of the row)."""
    p = np.full((1, 16), 121, dtype=np.uint8)
    p[0, :13] = np.arange(243, 256, dtype=np.uint8)
    _, bad = oracle.unpack_base3(p, 80)
    assert bad == 13
    _, bad = oracle.unpack_base3(p, 10)  # only bytes 0 and 1 hold codes
    assert bad == 2


@pytest.mark.parametrize("k", [1, 5, 16, 79, 80, 81, 2560, 6912])
def test_base3_roundtrip_and_row_size(k):
    """Random codes survive pack + unpack at every row length, rows take
    16 ceil(k / 80) bytes, and the pad digits are zeros (byte 121 past the codes)."""
    r = rng(k)
    c = r.integers(-1, 2, size=(6, k)).astype(np.int8)
    p = oracle.pack_base3(c)
    assert p.shape == (6, 16 * ((k + 79) // 80))
    back, bad = oracle.unpack_base3(p, k)
    assert bad == 0 and np.array_equal(back, c)
    full = (k + 4) // 5  # bytes that hold at least one code
    assert (p[:, full:] == 121).all()
    # the contraction is the same through either storage
    q = r.integers(-127, 128, size=(3, k)).astype(np.int8)
    two_bit = oracle.unpack(oracle.pack(c), k)[0] if k % 16 == 0 else c
    assert np.array_equal(oracle.contract(q, back), oracle.contract(q, two_bit))


# ------------------------------------------------------------------ O11 bfloat16
def _f32_from_bits(b):
    return np.array([b], dtype=np.uint32).view(np.float32)


def test_golden_bf16_round():
    for case in gold("bf16_round.json")["cases"]:
        x = _f32_from_bits(int(case["f32_bits"], 16))
        assert int(oracle.round_bf16(x)[0]) == int(case["bf16_bits"], 16), case


def _bf16_exact(v: float) -> int:
    """Nearest bfloat16 by exact rational arithmetic (ties to even), as bits."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                     # subnormals share the lowest exponent
    ulp = Fraction(2) ** (e - 7)         # 8 significant bits
    q, rem = divmod(a, ulp)
    q = int(q)
    if rem > ulp / 2 or (rem == ulp / 2 and q % 2 == 1):
        q += 1
    val = q * ulp
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = np.float32(float(val))            # exactly representable: 8 bits of mantissa
    return sign | (int(f.view(np.uint32)) >> 16)


def test_bf16_round_against_exact_rationals():
    r = rng(11)
    bits = r.integers(0, 2 ** 32, size=3000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    got = oracle.round_bf16(x)
    for v, g in zip(x.tolist(), got.tolist()):
        assert g == _bf16_exact(v), (v, hex(g))
    back = oracle.bf16_to_f32(got).view(np.uint32)  # widening is exact: the low 16 bits are zero
    assert np.array_equal(back >> 16, got.astype(np.uint32)) and not (back & 0xFFFF).any()


# ------------------------------------------------------------------ O12 final norm
def test_final_norm_scale_and_sign():
    """With eps = 0 the norm is exactly invariant to scaling by 2^j (ms scales by
    4^j, r by 2^-j, all exactly), and odd in x; a zero gain gives zeros."""
    r = rng(12)
    x = r.normal(size=(5, 96)).astype(np.float32)
    g = (1 + 0.1 * r.normal(size=96)).astype(np.float32)
    base = oracle.final_norm(x, g, eps=0.0)
    for j in (-3, 1, 5):
        assert np.array_equal(oracle.final_norm(np.ldexp(x, j).astype(np.float32), g, eps=0.0), base)
    neg = oracle.final_norm(-x, g, eps=0.0)
    assert np.array_equal(neg, base ^ np.uint16(0x8000))
    assert not (oracle.final_norm(x, np.zeros(96, np.float32)) & np.uint16(0x7FFF)).any()


def test_final_norm_against_exact_rationals():
    """A few rows computed with exact rationals and 60-digit decimals, following
    R20 step by step: ms exact, r = nearest float32 to 1/sqrt(ms + eps), then two
    float32 products and one bfloat16 rounding."""
    getcontext().prec = 60
    r = rng(13)
    x = r.normal(size=(3, 16)).astype(np.float32)
    g = (1 + 0.1 * r.normal(size=16)).astype(np.float32)
    eps = np.float32(1e-5)
    got = oracle.final_norm(x, g, eps=float(eps))
    for i in range(3):
        ms = sum(Fraction(float(v)) ** 2 for v in x[i]) / 16
        d = Decimal(ms.numerator) / Decimal(ms.denominator) + Decimal(float(eps))
        rr = np.float32(float(1 / d.sqrt()))
        for j in range(16):
            v = np.float32(x[i, j] * rr)
            o = np.float32(g[j] * v)
            assert int(got[i, j]) == _bf16_exact(float(o))


# ------------------------------------------------------------------ O13 head
def test_lm_head_against_exact_rationals():
    r = rng(14)
    o = oracle.round_bf16(r.normal(size=(3, 40)).astype(np.float32))
    w = oracle.round_bf16((0.02 * r.normal(size=(7, 40))).astype(np.float32))
    y, a = oracle.lm_head(o, w)
    of, wf = oracle.bf16_to_f32(o), oracle.bf16_to_f32(w)
    for i in range(3):
        for j in range(7):
            exact = sum(Fraction(float(of[i, t])) * Fraction(float(wf[j, t])) for t in range(40))
            assert y[i, j] == np.float32(float(exact))
            assert a[i, j] >= abs(float(exact))


def test_lm_head_one_hot_rows_select_columns():
    """A head row that is one-hot at column t returns o[:, t] exactly."""
    r = rng(15)
    o = oracle.round_bf16(r.normal(size=(4, 32)).astype(np.float32))
    w = np.zeros((32, 32), dtype=np.uint16)
    w[np.arange(32), np.arange(32)] = 0x3F80  # 1.0
    y, _ = oracle.lm_head(o, w)
    assert np.array_equal(y, oracle.bf16_to_f32(o))


# ------------------------------------------------------------------ O14 RoPE (R19)
def test_golden_rope():
    g = gold("rope.json")
    for case in g["cases"]:
        x = np.array([case["x"]], dtype=np.float32)
        y = oracle.rope(x, [g["position"]], 1, g["head_dim"], g["theta"])
        assert np.array_equal(y[0], np.array(case["y"], dtype=np.float32)), (case, y)


def test_rope_position_zero_is_identity_and_pairs_keep_length():
    r = rng(16)
    x = r.normal(size=(3, 2 * 128)).astype(np.float32)
    assert np.array_equal(oracle.rope(x, [0, 0, 0], 2, 128, 5e5), x)
    # outside the rotary's 4096 positions the angle is 0 (reading R19)
    assert np.array_equal(oracle.rope(x, [-1, 4096, 10 ** 9], 2, 128, 5e5), x)
    y = oracle.rope(x, [1, 517, 4095], 2, 128, 5e5).astype(np.float64).reshape(3, 2, 2, 64)
    xx = x.astype(np.float64).reshape(3, 2, 2, 64)
    n0 = xx[:, :, 0] ** 2 + xx[:, :, 1] ** 2
    n1 = y[:, :, 0] ** 2 + y[:, :, 1] ** 2
    assert np.allclose(n1, n0, rtol=2e-6, atol=1e-30)


def test_rope_scores_depend_on_relative_position():
    """<rope(q, a), rope(k, b)> is a function of a - b: shifting both positions by
    the same amount keeps every head's score (to fp32 rounding)."""
    r = rng(17)
    q = r.normal(size=(1, 128)).astype(np.float32)
    k = r.normal(size=(1, 128)).astype(np.float32)
    base = None
    for a, b in ((7, 3), (107, 103), (2007, 2003)):
        s = float(np.dot(oracle.rope(q, [a], 1, 128, 5e5)[0].astype(np.float64),
                         oracle.rope(k, [b], 1, 128, 5e5)[0].astype(np.float64)))
        if base is None:
            base = s
        assert abs(s - base) <= 1e-4 * float(np.abs(q).sum() * np.abs(k).max()), (a, b, s, base)


# ------------------------------------------------------------------ O15 attention (R21)
def _caches(r, n_slots, n_kv, tmax, hd, scale=1.0):
    kc = oracle.round_bf16((scale * r.normal(size=(n_slots, n_kv, tmax, hd))).astype(np.float32))
    vc = oracle.round_bf16(r.normal(size=(n_slots, n_kv, tmax, hd)).astype(np.float32))
    return kc, vc


def test_attention_single_position_returns_the_value():
    r = rng(18)
    kc, vc = _caches(r, 2, 2, 8, 16)
    q = r.normal(size=(2, 4 * 16)).astype(np.float32)
    out, _, _, bad = oracle.attention(q, kc, vc, [1, 0], [0, 0], 4, 2, 16)
    assert bad == 0
    for t, s in enumerate((1, 0)):
        for h in range(4):
            assert np.array_equal(out[t, 16 * h:16 * h + 16], oracle.bf16_to_f32(vc[s, h // 2, 0]))


def test_attention_equal_keys_average_and_heads_share_kv():
    """Equal keys give equal weights: the output is the mean of the values. Values
    that are constant per key/value head show which head each query head reads."""
    n_heads, n_kv, hd, T = 8, 2, 8, 5
    kc = np.zeros((1, n_kv, 16, hd), dtype=np.uint16)
    kc[...] = oracle.round_bf16(np.full(hd, 0.5, np.float32))
    vc = oracle.round_bf16(np.random.default_rng(1).normal(size=(1, n_kv, 16, hd)).astype(np.float32))
    q = np.random.default_rng(2).normal(size=(1, n_heads * hd)).astype(np.float32)
    out, _, _, _ = oracle.attention(q, kc, vc, [0], [T - 1], n_heads, n_kv, hd)
    vf = oracle.bf16_to_f32(vc).astype(np.float64)
    for h in range(n_heads):
        want = vf[0, h // (n_heads // n_kv), :T].mean(axis=0)
        assert np.allclose(out[0, h * hd:(h + 1) * hd], want, rtol=1e-6, atol=1e-7)
    const = np.zeros_like(vc)
    for g in range(n_kv):
        const[0, g] = oracle.round_bf16(np.full(hd, g + 1.0, np.float32))
    out2, _, _, _ = oracle.attention(q, oracle.round_bf16(np.random.default_rng(3).normal(
        size=(1, n_kv, 16, hd)).astype(np.float32)), const, [0], [9], n_heads, n_kv, hd)
    for h in range(n_heads):
        assert np.all(out2[0, h * hd:(h + 1) * hd] == np.float32(h // (n_heads // n_kv) + 1))


def test_golden_attention_scale():
    """[nnterp] "Loading" and "Config": two keys with hand-worked softmax weights
    under the 1/sqrt(head_dim) score scale (tests/golden/attention_scale.json);
    dropping or squaring the scale moves the weights far outside the bound."""
    g = gold("attention_scale.json")
    bf = {2.0: 0x4000, 16.0: 0x4180, 1.0: 0x3F80}  # bfloat16 bit patterns of exact values
    for case in g["cases"]:
        hd = case["head_dim"]
        kc = np.zeros((1, 1, 2, hd), dtype=np.uint16)
        vc = np.zeros((1, 1, 2, hd), dtype=np.uint16)
        kc[0, 0, 1, 0] = bf[case["key1_dim0"]]
        vc[0, 0, 0, 0] = bf[1.0]
        vc[0, 0, 1, 1] = bf[1.0]
        q = np.zeros((1, hd), dtype=np.float32)
        q[0, 0] = 1.0
        out, _, _, bad = oracle.attention(q, kc, vc, [0], [1], 1, 1, hd)
        assert bad == 0
        want = np.zeros(hd)
        want[0], want[1] = case["out_dim0"], case["out_dim1"]
        # the only rounding is the final one to fp32
        assert np.all(np.abs(out[0].astype(np.float64) - want) <= 2.0 ** -24 * np.abs(want) + 1e-300), (hd, out[0, :2])


def test_golden_kv_append_layout():
    """[nnterp] "Config" and "Loading"; reading R21: [slot][kv head][position][hd]
    bfloat16 caches, out-of-range tokens skipped (tests/golden/kv_append_layout.json)."""
    g = gold("kv_append_layout.json")
    ns, nkv, tmax, hd = g["n_slots"], g["n_kv"], g["t_max"], g["head_dim"]
    keys = np.array([[float.fromhex(v) if isinstance(v, str) else float(v) for v in row] for row in g["keys"]],
                    dtype=np.float32)
    kc = np.full((ns, nkv, tmax, hd), g["sentinel"], dtype=np.uint16)
    vc = kc.copy()
    skipped = oracle.kv_append(kc, vc, keys, -keys, g["slot"], g["pos"], nkv, hd)
    assert skipped == 3
    want_k = np.full(kc.size, g["sentinel"], dtype=np.uint16)
    want_v = want_k.copy()
    for off, bits in g["expect_k_hex"].items():
        want_k[int(off):int(off) + hd] = [int(b, 16) for b in bits]
    for off, bits in g["expect_v_hex"].items():
        want_v[int(off):int(off) + hd] = [int(b, 16) for b in bits]
    assert np.array_equal(kc.reshape(-1), want_k)
    assert np.array_equal(vc.reshape(-1), want_v)


def test_golden_rescale_order():
    """[nnterp] "The two checkpoints"; reading R10: the per-token factor first, then
    gamma (tests/golden/rescale_order.json); the other order, or one rounding of
    the exact product, gives a different fp32 value on this case."""
    g = gold("rescale_order.json")
    deq = np.array([float.fromhex(g["deq"])], dtype=np.float32)
    gam = float.fromhex(g["gamma"])
    y = oracle.rescale(np.array([[g["acc"]]], dtype=np.int32), deq, [gam], [1])
    assert float(y[0, 0]) == float.fromhex(g["y"])
    assert float.fromhex(g["y"]) != float.fromhex(g["y_other_order"])


def test_attention_permutation_dominance_and_range():
    r = rng(19)
    kc, vc = _caches(r, 1, 1, 32, 16)
    q = r.normal(size=(1, 16)).astype(np.float32)
    out, _, _, _ = oracle.attention(q, kc, vc, [0], [20], 1, 1, 16)
    perm = r.permutation(21)
    kp, vp = kc.copy(), vc.copy()
    kp[0, 0, :21], vp[0, 0, :21] = kc[0, 0, perm], vc[0, 0, perm]
    outp, _, _, _ = oracle.attention(q, kp, vp, [0], [20], 1, 1, 16)
    assert np.allclose(outp, out, rtol=1e-12, atol=1e-12)
    # a key along q with a score 40 above the rest takes all the weight
    kd = kc.copy()
    kd[0, 0, :21] = 0
    kd[0, 0, 7] = oracle.round_bf16((q[0] * (40.0 * 4.0 / float(np.dot(q[0], q[0])))).astype(np.float32))
    outd, _, _, _ = oracle.attention(q, kd, vc, [0], [20], 1, 1, 16)
    assert np.allclose(outd[0], oracle.bf16_to_f32(vc[0, 0, 7]), rtol=1e-12, atol=1e-12)
    outb, _, _, bad = oracle.attention(np.vstack([q, q, q]), kc, vc, [0, 1, 0], [3, 3, 32], 1, 1, 16)
    assert bad == 2 and not outb[1:].any()


# ------------------------------------------------------------------ O4
def test_golden_act_codes():
    """[nnterp] "The projections quantize their inputs and weights": round(x * 127 / max|x|)."""
    for case in gold("act_codes.json")["cases"]:
        x = np.array([case["x"]], dtype=np.float32)
        q, deq = oracle.quant_absmax(x)
        assert q.tolist() == [case["codes"]]
        assert deq[0] == np.float32(float(Fraction(case["deq_num"], case["deq_den"])))


def _round_half_even(fr: Fraction) -> int:
    fl = math.floor(fr)
    d = fr - fl
    if d > Fraction(1, 2):
        return fl + 1
    if d < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def test_P5_codes_against_exact_rationals():
    """q = round_half_even(x * 127 / a) exactly, except where x * 127 / a lies within
    the fp32 rounding of the scale and product (2^-22 relative) of a half-integer;
    there q is one of the two neighbours. Also |q| <= 127, max|q| = 127, q(-x) = -q(x)."""
    r = rng(6)
    x = synth.activations(synth.stream_seed(8, tensor=synth.T_ACT), 48, 64, n_outliers=2)
    x[3] = 0.0
    x[5, :] = (r.integers(-40, 41, size=64) / 8.0).astype(np.float32)  # grid values: many exact ties
    q, deq = oracle.quant_absmax(x)
    qn, deqn = oracle.quant_absmax(-x)
    assert np.array_equal(qn, -q) and np.array_equal(deqn, deq)
    assert np.abs(q.astype(int)).max() <= 127
    near = 0
    for i in range(x.shape[0]):
        a = Fraction(float(np.abs(x[i]).max()))
        if a == 0:
            assert not q[i].any() and deq[i] == 0
            continue
        assert np.abs(q[i].astype(int)).max() == 127
        assert deq[i] == np.float32(float(a / 127))
        for j in range(x.shape[1]):
            t = Fraction(float(x[i, j])) * 127 / a
            want = _round_half_even(t)
            if int(q[i, j]) != want:
                frac = abs(t - math.floor(t) - Fraction(1, 2))
                assert frac <= abs(t) * Fraction(1, 2 ** 22) and abs(int(q[i, j]) - t) < 1, (i, j)
                near += 1
    assert near <= 4


def test_P5_tiny_amax_rows():
    """Rows whose max|x| is tiny (down to subnormals, where 127 / a overflows fp32) are
    quantized like the same row scaled by a power of two: codes are scale invariant
    (the per-token scale cancels), deq = a / 127 rounded to fp32."""
    base = synth.activations(synth.stream_seed(9, tensor=synth.T_ACT), 6, 32)
    for e in (-100, -120, -126, -130, -140):
        x = (base.astype(np.float64) * 2.0 ** e).astype(np.float32)
        # keep rows exactly representable: compare against the same fp32 values scaled up
        up = (x.astype(np.float64) * 2.0 ** (-e)).astype(np.float32)
        assert np.array_equal((up.astype(np.float64) * 2.0 ** e).astype(np.float32), x)
        q, deq = oracle.quant_absmax(x)
        qu, _ = oracle.quant_absmax(up)
        assert np.array_equal(q, qu), e
        a = np.abs(x).max(axis=1).astype(np.float64)
        want = np.array([float(Fraction(float(v)) / 127) for v in a]).astype(np.float32)
        assert np.array_equal(deq, want)


@pytest.mark.parametrize("j", [-20, -3, 1, 7, 30])
def test_P6_power_of_two_scaling(j):
    """[nnterp] "Scaling inside a sublayer is undone by the sub-norm": x -> 2^j x leaves the
    codes identical and scales deq by exactly 2^j."""
    x = synth.activations(synth.stream_seed(10, tensor=synth.T_ACT), 16, 96, n_outliers=1)
    q, deq = oracle.quant_absmax(x)
    xs = (x * np.float32(2.0 ** j)).astype(np.float32)
    q2, deq2 = oracle.quant_absmax(xs)
    assert np.array_equal(q, q2)
    assert np.array_equal(deq2, (deq * np.float32(2.0 ** j)).astype(np.float32))


# ------------------------------------------------------------------ O5
def _exact_rms_deq(a, xs, eps32, gain=None):
    getcontext().prec = 60
    k = len(xs)
    ms = sum(Decimal(float(v)) ** 2 for v in xs) / k
    r = (ms + Decimal(float(eps32))).sqrt()
    return float(Decimal(float(a)) / 127 / r)


@pytest.mark.parametrize("c", [2.0, -0.37, 1e-3, 150.0])
def test_P7_constant_row_closed_form(c):
    """RMSNorm(x) = g x / sqrt(mean(x^2) + eps) with eps 1e-5 ([nnterp] "Config",
    "The block, in order"). A constant row c quantizes to +-127 everywhere and
    deq = |c| / 127 / sqrt(c^2 + eps)."""
    k = 64
    x = np.full((1, k), c, dtype=np.float32)
    q, deq = oracle.quant_rms(x, None, 1e-5)
    assert np.all(q == (127 if c > 0 else -127))
    want = _exact_rms_deq(abs(np.float32(c)), x[0], np.float32(1e-5))
    assert abs(float(deq[0]) - want) <= 0.5 * F32_ULP * abs(want) * 1.0001


def test_P7_random_rows_closed_form_and_doubling():
    """deq of random rows against a 60-digit evaluation of |max g x| / 127 / sqrt(ms + eps);
    doubling x keeps the codes and changes deq by 2 sqrt(ms + eps) / sqrt(4 ms + eps)."""
    x = synth.activations(synth.stream_seed(11, tensor=synth.T_ACT), 12, 160, n_outliers=2)
    gain = (1.0 + 0.1 * synth.normal_f32(synth.stream_seed(11, tensor=synth.T_GAIN), 160)).astype(np.float32)
    for g in (None, gain):
        q, deq = oracle.quant_rms(x, g, 1e-5)
        q2, deq2 = oracle.quant_rms((2 * x).astype(np.float32), g, 1e-5)
        assert np.array_equal(q, q2)
        v = x if g is None else (g * x).astype(np.float32)
        q_abs, _ = oracle.quant_absmax(v)
        assert np.array_equal(q, q_abs)  # the codes are those of g * x: 1/r cancels
        for i in range(x.shape[0]):
            want = _exact_rms_deq(np.abs(v[i]).max(), x[i], np.float32(1e-5))
            assert abs(float(deq[i]) - want) <= 0.5 * F32_ULP * want * 1.0001
            want2 = _exact_rms_deq(np.abs(2 * v[i]).max(), 2 * x[i], np.float32(1e-5))
            assert abs(float(deq2[i]) - want2) <= 0.5 * F32_ULP * want2 * 1.0001


def test_P7_matches_literal_normalize_then_round():
    """The scale-invariant codes equal the literal order (normalize in fp64, then
    round(n * 127 / max|n|)) except at near-ties of the fp32 order."""
    x = synth.activations(synth.stream_seed(12, tensor=synth.T_ACT), 64, 256, n_outliers=3)
    q, _ = oracle.quant_rms(x, None, 1e-5)
    x64 = x.astype(np.float64)
    r = np.sqrt((x64 ** 2).mean(axis=1, keepdims=True) + float(np.float32(1e-5)))
    n = x64 / r
    t = n * 127.0 / np.abs(n).max(axis=1, keepdims=True)
    lit = np.rint(t)
    diff = lit != q
    assert diff.sum() <= 4
    assert np.all(np.abs(np.abs(t[diff] - np.floor(t[diff])) - 0.5) < 1e-4)


# ------------------------------------------------------------------ O6
def test_golden_relu2():
    """[nnterp] "The MLP gates with a squared ReLU": relu(gate)^2 * up, zero where gate <= 0."""
    cases = gold("relu2.json")["cases"]
    gu = np.array([[c["gate"] for c in cases] + [c["up"] for c in cases]], dtype=np.float32)
    out = oracle.relu2_mul(gu, len(cases))
    assert out.ravel().tolist() == [c["out"] for c in cases]


def test_P8a_nonpositive_gate_gives_zero_code():
    """Wherever the gate is <= 0 the product and its code are exactly 0."""
    m, inter = 16, 192
    g = synth.activations(synth.stream_seed(13, tensor=synth.T_ACT), m, inter)
    u = synth.activations(synth.stream_seed(13, tensor=synth.T_ACT2), m, inter)
    g[0, :5] = -0.0
    mi = oracle.relu2_mul(np.concatenate([g, u], axis=1), inter)
    assert np.all(mi[g <= 0] == 0)
    assert np.all(mi[g > 0] != 0)
    q, _ = oracle.quant_rms(mi, None, 1e-5)
    assert np.all(q[g <= 0] == 0)
    assert 0.4 < (g <= 0).mean() < 0.6


# ------------------------------------------------------------------ O7
def test_P9_brute_force_every_ternary_row():
    """Every ternary row of length <= 6 against random int8 codes, compared with an
    int64 matrix product (a library routine)."""
    r = rng(14)
    for k in range(1, 7):
        rows = np.array(np.meshgrid(*[[-1, 0, 1]] * k, indexing="ij")).reshape(k, -1).T.astype(np.int8)
        q = r.integers(-127, 128, size=(5, k), dtype=np.int8)
        acc = oracle.contract(q, rows)
        assert np.array_equal(acc, q.astype(np.int64) @ rows.astype(np.int64).T)


def test_P9_closed_forms():
    """all q = 127, c = +1 -> 127 K; alternating +-1 against constant q -> 0;
    one-hot rows copy columns of q; K = 6912 bound fits int32."""
    k = 6912
    q = np.full((2, k), 127, dtype=np.int8)
    c = np.ones((3, k), dtype=np.int8)
    c[1, 1::2] = -1
    c[2] = -1
    acc = oracle.contract(q, c)
    assert acc[:, 0].tolist() == [127 * k] * 2 and acc[:, 1].tolist() == [0, 0] and acc[:, 2].tolist() == [-127 * k] * 2
    r = rng(15)
    q = r.integers(-127, 128, size=(7, 48), dtype=np.int8)
    sel = r.permutation(48)[:10]
    onehot = np.zeros((10, 48), dtype=np.int8)
    onehot[np.arange(10), sel] = 1
    assert np.array_equal(oracle.contract(q, onehot), q[:, sel].astype(np.int32))
    assert np.array_equal(oracle.contract(q, -onehot), -q[:, sel].astype(np.int32))


# ------------------------------------------------------------------ O8
def test_P10_rescale_equals_dequantized_linear_map():
    """[nnterp] "The projections quantize their inputs and weights": the projection's
    output is the exact product of the quantized input and the ternary weights. In fp64,
    y64 = (q * deq) @ (c * gamma)^T; the fp32 result is within 3 * 2^-24 |y| of it."""
    x = synth.activations(synth.stream_seed(16, tensor=synth.T_ACT), 32, 256, n_outliers=3)
    w = synth.weights(synth.stream_seed(16, tensor=synth.T_WEIGHT), 96, 256)
    wu = synth.weights(synth.stream_seed(17, tensor=synth.T_WEIGHT), 80, 256, sigma=0.05)
    g1, g2 = oracle.absmean(w), oracle.absmean(wu)
    c = np.concatenate([oracle.ternarize(w, g1), oracle.ternarize(wu, g2)])
    out = oracle.forward(x, c, [g1, g2], [96, 176])
    q, deq = out["q"], out["deq"]
    gam = np.concatenate([np.full(96, float(np.float32(g1))), np.full(80, float(np.float32(g2)))])
    y64 = (q.astype(np.float64) * deq.astype(np.float64)[:, None]) @ (c.astype(np.float64) * gam[:, None]).T
    y = out["y"].astype(np.float64)
    # the fp64 evaluation of y64 has its own error, at most ~K 2^-53 sum|terms|
    mag = (np.abs(q).astype(np.float64) * deq.astype(np.float64)[:, None]) @ (np.abs(c).astype(np.float64) * gam[:, None]).T
    assert np.all(np.abs(y - y64) <= 3 * 2.0 ** -24 * np.abs(y64) + 2 * x.shape[1] * 2.0 ** -53 * mag)
    assert np.all((y == 0) == (out["acc"] == 0))
    # fused == unfused, bit for bit
    a = oracle.forward(x, c[:96], [g1])["y"]
    b = oracle.forward(x, c[96:], [g2])["y"]
    assert np.array_equal(out["y"], np.concatenate([a, b], axis=1))


# ------------------------------------------------------------------ O9 / O10
def _literal_quant(v):
    """round(v * 127 / max|v|) in fp64 and its dequantized value (pages' formula)."""
    a = np.abs(v).max(axis=1, keepdims=True)
    a = np.where(a == 0, 1.0, a)
    q = np.clip(np.rint(v * 127.0 / a), -127, 127)
    return q * a / 127.0


def _literal_rms(v, eps):
    return v / np.sqrt((v ** 2).mean(axis=1, keepdims=True) + eps)


def _literal_linear(v, c, gam):
    return _literal_quant(v) @ (c.astype(np.float64) * gam[:, None]).T


def test_ffn_block_against_literal_fp64_formulation():
    """O9 against the block written straight from [nnterp] "The block, in order" in
    fp64 (normalize, round, dequantize, matmul): equal up to fp32 rounding."""
    m, hdim, inter = 24, 64, 96
    x = synth.activations(synth.stream_seed(18, tensor=synth.T_ACT), m, hdim)
    wg = synth.weights(synth.stream_seed(18, 0, 1, synth.T_WEIGHT), inter, hdim)
    wu = synth.weights(synth.stream_seed(18, 0, 2, synth.T_WEIGHT), inter, hdim)
    wd = synth.weights(synth.stream_seed(18, 0, 3, synth.T_WEIGHT), hdim, inter)
    gg, gu_, gd = oracle.absmean(wg), oracle.absmean(wu), oracle.absmean(wd)
    cg, cu, cd = oracle.ternarize(wg, gg), oracle.ternarize(wu, gu_), oracle.ternarize(wd, gd)
    out = oracle.ffn_block(x, np.concatenate([cg, cu]), [gg, gu_], cd, gd, None, 1e-5)
    eps = float(np.float32(1e-5))
    x64 = x.astype(np.float64)
    G = _literal_linear(x64, cg, np.full(inter, gg))
    U = _literal_linear(x64, cu, np.full(inter, gu_))
    Mi = np.maximum(G, 0) ** 2 * U
    Y = _literal_linear(_literal_rms(Mi, eps), cd, np.full(hdim, gd))
    scale = np.abs(Y).max()
    assert np.abs(out["y"] - Y).max() <= 1e-4 * scale
    assert np.array_equal(out["gu"][:, :inter] <= 0, G <= 0) or np.mean((out["gu"][:, :inter] <= 0) != (G <= 0)) < 1e-3


def _small_decoder_weights(seed, hdim, inter, nh, nkv, hd, zero=()):
    kvd = nkv * hd
    shapes = {"q": (hdim, hdim), "k": (kvd, hdim), "v": (kvd, hdim), "o": (hdim, hdim),
              "gate": (inter, hdim), "up": (inter, hdim), "down": (hdim, inter)}
    codes, gam = {}, {}
    for i, (name, (n, k)) in enumerate(shapes.items()):
        w = synth.weights(synth.stream_seed(seed, 5, i, synth.T_WEIGHT), n, k)
        if name in zero:
            w[:] = 0
        gam[name] = oracle.absmean(w)
        codes[name] = oracle.ternarize(w, gam[name])
    return {"qkv": np.concatenate([codes["q"], codes["k"], codes["v"]]), "g_qkv": [gam["q"], gam["k"], gam["v"]],
            "o": codes["o"], "g_o": gam["o"], "gu": np.concatenate([codes["gate"], codes["up"]]),
            "g_gu": [gam["gate"], gam["up"]], "down": codes["down"], "g_down": gam["down"]}, codes, gam


def test_decoder_layer_against_literal_fp64_formulation():
    """O10 against [nnterp] "The block, in order" written out in fp64: pre-norm, q/k/v,
    self-only attention (query head h reads key/value head h // 4, section "Loading"),
    attn_sub_norm, o, residual, pre-norm, gate/up, relu^2, ffn_sub_norm, down, residual."""
    hdim, inter, nh, nkv, hd, m = 64, 96, 8, 2, 8, 6
    w, codes, gam = _small_decoder_weights(19, hdim, inter, nh, nkv, hd)
    x = synth.activations(synth.stream_seed(19, tensor=synth.T_ACT), m, hdim)
    out = oracle.decoder_layer(x, w, 1e-5, nh, nkv, hd)
    eps = float(np.float32(1e-5))
    lin = lambda v, name: _literal_linear(v, codes[name], np.full(codes[name].shape[0], gam[name]))
    x64 = x.astype(np.float64)
    z = _literal_rms(x64, eps)
    V = lin(z, "v")
    A = np.concatenate([V[:, (h // (nh // nkv)) * hd:(h // (nh // nkv) + 1) * hd] for h in range(nh)], axis=1)
    H = x64 + lin(_literal_rms(A, eps), "o")
    z2 = _literal_rms(H, eps)
    Mi = np.maximum(lin(z2, "gate"), 0) ** 2 * lin(z2, "up")
    X1 = H + lin(_literal_rms(Mi, eps), "down")
    assert np.abs(out["h"] - H).max() <= 1e-4 * np.abs(H).max()
    assert np.abs(out["x"] - X1).max() <= 1e-4 * np.abs(X1).max()


def test_P11_P12_residual_wiring_and_head_map():
    """[nnterp] identity layer_input + attention_output + mlp_output == layer_output,
    and "an edit to key/value head j reaches query heads 4j to 4j + 3"."""
    hdim, inter, nh, nkv, hd, m = 64, 96, 8, 2, 8, 4
    x = synth.activations(synth.stream_seed(20, tensor=synth.T_ACT), m, hdim)
    w0, _, _ = _small_decoder_weights(20, hdim, inter, nh, nkv, hd, zero=("o", "down"))
    out = oracle.decoder_layer(x, w0, 1e-5, nh, nkv, hd)
    assert np.array_equal(out["h"], x) and np.array_equal(out["x"], x)
    w1, _, _ = _small_decoder_weights(20, hdim, inter, nh, nkv, hd, zero=("v",))
    out1 = oracle.decoder_layer(x, w1, 1e-5, nh, nkv, hd)
    assert np.array_equal(out1["h"], x)  # zero values -> zero attention -> zero o_proj output
    w2, _, _ = _small_decoder_weights(20, hdim, inter, nh, nkv, hd)
    out2 = oracle.decoder_layer(x, w2, 1e-5, nh, nkv, hd)
    h = (x + out2["o"]["y"]).astype(np.float32)
    assert np.array_equal(out2["x"], (h + out2["down"]["y"]).astype(np.float32))
    # head map: an edit of key/value head j changes exactly query heads 4j .. 4j+3
    v = np.arange(m * nkv * hd, dtype=np.float32).reshape(m, nkv * hd)
    a = oracle.gqa_broadcast(v, nh, nkv, hd)
    for j in range(nkv):
        v2 = v.copy()
        v2[:, j * hd:(j + 1) * hd] += 1000
        changed = np.any(oracle.gqa_broadcast(v2, nh, nkv, hd) != a, axis=0).reshape(nh, hd).any(axis=1)
        grp = nh // nkv
        assert changed.tolist() == [grp * j <= hh < grp * (j + 1) for hh in range(nh)]
