"""CPU oracle for the BitNet b1.58 BitLinear hot path — TEST INFRASTRUCTURE.

The reference that the HIP library is checked against. Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it; the library itself never does, and fails loudly when its own HIP build is
missing instead of falling back to anything here.

The steps live in ``bitlinear_oracle.c`` (plain C, one function per step, each
citing the passage it follows). This module loads that library, marshals numpy
arrays, and composes the two block-level chains:

* :func:`ffn_block` — the MLP of the nnterp BitNet page, section "The block, in
  order" (``m = relu(gate(z))**2 * up(z)``, ``out = down(ffn_sub_norm(m))``),
  taken without pre-norm or residual (reading R13);
* :func:`decoder_layer` — one decoder block's projections in the order of that
  section, with the attention replaced by its exact value when every token
  attends only to itself (reading R12): the output of query head ``h`` is the
  value of key/value head ``h // (n_heads / n_kv_heads)`` (section "Loading":
  20 query heads share 5 key/value heads).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run oracle/build.py (or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        sig = {
            "orc_absmean": (ctypes.c_double, [_p, _i64]),
            "orc_ternarize": (None, [_p, _i64, ctypes.c_double, _p]),
            "orc_pack": (ctypes.c_int, [_p, _i64, _i64, _p]),
            "orc_unpack": (_i64, [_p, _i64, _i64, _p]),
            "orc_round_bf16": (None, [_p, _i64, _p]),
            "orc_bf16_to_f32": (None, [_p, _i64, _p]),
            "orc_final_norm": (None, [_p, _i64, _i64, _p, ctypes.c_float, _p]),
            "orc_lm_head": (None, [_p, _i64, _i64, _p, _i64, _p, _p]),
            "orc_rope": (None, [_p, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _p, ctypes.c_double, _i64]),
            "orc_attention": (_i64, [_p, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _p, _p, _i64, _i64,
                                     _p, _p, _p, _p, _p, _p]),
            "orc_base3_row_bytes": (_i64, [_i64]),
            "orc_pack_base3": (ctypes.c_int, [_p, _i64, _i64, _p]),
            "orc_unpack_base3": (_i64, [_p, _i64, _i64, _p]),
            "orc_quant_absmax": (None, [_p, _i64, _i64, _p, _p]),
            "orc_quant_rms": (None, [_p, _i64, _i64, _p, ctypes.c_float, _p, _p, _p]),
            "orc_relu2_mul": (None, [_p, _i64, _i64, _p]),
            "orc_contract": (ctypes.c_int, [_p, _i64, _i64, _p, _i64, _p]),
            "orc_rescale": (None, [_p, _i64, _i64, _p, _p, _p, ctypes.c_int, _p]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


# ---------------------------------------------------------------- single steps
def absmean(w) -> float:
    """O1: gamma = mean |W| (fp64, sequential)."""
    w, pw = _c(w, np.float32)
    return float(_load().orc_absmean(pw, w.size))


def ternarize(w, gamma: float) -> np.ndarray:
    """O2: codes in {-1, 0, 1}: sign(W) where |W| > gamma / 2."""
    w, pw = _c(w, np.float32)
    c = np.empty(w.shape, dtype=np.int8)
    _load().orc_ternarize(pw, w.size, float(gamma), c.ctypes.data)
    return c


def pack(c) -> np.ndarray:
    """O3: [n][k] codes -> [n][k/4] bytes (four to a byte)."""
    c, pc = _c(c, np.int8)
    n, k = c.shape
    p = np.empty((n, k // 4), dtype=np.uint8)
    if _load().orc_pack(pc, n, k, p.ctypes.data) != 0:
        raise ValueError("pack: k must be a multiple of 16 and codes in {-1, 0, 1}")
    return p


def unpack(p, k: int):
    """O3 inverse: returns (codes [n][k], number of invalid fields)."""
    p, pp = _c(p, np.uint8)
    n = p.shape[0]
    c = np.empty((n, k), dtype=np.int8)
    bad = _load().orc_unpack(pp, n, k, c.ctypes.data)
    if bad < 0:
        raise ValueError("unpack: k must be a multiple of 16")
    return c, int(bad)


def base3_row_bytes(k: int) -> int:
    """Bytes of one row of k codes stored five to a byte (16 per 80 codes)."""
    return int(_load().orc_base3_row_bytes(k))


def pack_base3(c) -> np.ndarray:
    """Five codes to a byte: [n][k] codes -> [n][16 ceil(k / 80)] base-3 bytes."""
    c, pc = _c(c, np.int8)
    n, k = c.shape
    p = np.empty((n, base3_row_bytes(k)), dtype=np.uint8)
    if _load().orc_pack_base3(pc, n, k, p.ctypes.data) != 0:
        raise ValueError("pack_base3: codes must be in {-1, 0, 1}")
    return p


def unpack_base3(p, k: int):
    """Inverse of :func:`pack_base3`: returns (codes [n][k], number of invalid bytes)."""
    p, pp = _c(p, np.uint8)
    n = p.shape[0]
    assert p.shape[1] == base3_row_bytes(k)
    c = np.empty((n, k), dtype=np.int8)
    bad = _load().orc_unpack_base3(pp, n, k, c.ctypes.data)
    return c, int(bad)


def round_bf16(x) -> np.ndarray:
    """O11: fp32 -> bfloat16 bit patterns (uint16), nearest, ties to even."""
    x, px = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_round_bf16(px, x.size, out.ctypes.data)
    return out


def bf16_to_f32(b) -> np.ndarray:
    """bfloat16 bit patterns -> their fp32 values (exact)."""
    b, pb = _c(b, np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    _load().orc_bf16_to_f32(pb, b.size, out.ctypes.data)
    return out


def final_norm(x, gain=None, eps: float = 1e-5) -> np.ndarray:
    """O12: the final RMSNorm of [m][k] fp32 rows, as bfloat16 bits [m][k] (R20)."""
    x, px = _c(x, np.float32)
    m, k = x.shape
    pg = None
    if gain is not None:
        gain, pg = _c(gain, np.float32)
    out = np.empty((m, k), dtype=np.uint16)
    _load().orc_final_norm(px, m, k, pg, eps, out.ctypes.data)
    return out


def lm_head(o, w):
    """O13: logits [m][n] fp32 of bfloat16 inputs o [m][k] and head w [n][k]
    (both uint16 bit patterns), and sum |o w| per logit (fp64)."""
    o, po = _c(o, np.uint16)
    w, pw = _c(w, np.uint16)
    m, k = o.shape
    n = w.shape[0]
    assert w.shape[1] == k
    y = np.empty((m, n), dtype=np.float32)
    a = np.empty((m, n), dtype=np.float64)
    _load().orc_lm_head(po, m, k, pw, n, y.ctypes.data, a.ctypes.data)
    return y, a


def rope(x, pos, n_heads: int, head_dim: int, theta: float, col0: int = 0, n_pos: int = 4096) -> np.ndarray:
    """O14 (R19): rotate-half RoPE of the n_heads head vectors starting at column
    col0 of each row of x [m][ld], token r at position pos[r]; positions outside
    [0, n_pos) turn by angle 0. Returns a copy."""
    y = np.array(x, dtype=np.float32, order="C", copy=True)
    m, ld = y.shape
    p, pp = _c(np.asarray(pos, dtype=np.int64), np.int64)
    _load().orc_rope(y.ctypes.data, m, ld, col0, n_heads, head_dim, pp, theta, n_pos)
    return y


def attention(q, k_cache, v_cache, slot, pos, n_heads: int, n_kv: int, head_dim: int):
    """O15 (R21): each token's attention over positions 0..pos of its slot.
    q [m][ldq] fp32 (heads from column 0); caches [n_slots][n_kv][t_max][hd]
    bfloat16 bits. Returns (out [m][n_heads hd] fp32, vmag, smag [m][n_heads],
    number of tokens out of range)."""
    q, pq = _c(q, np.float32)
    kc, pk = _c(k_cache, np.uint16)
    vc, pv = _c(v_cache, np.uint16)
    n_slots, _, tmax, _ = kc.shape
    m = q.shape[0]
    sl, ps = _c(np.asarray(slot, dtype=np.int64), np.int64)
    po, pp = _c(np.asarray(pos, dtype=np.int64), np.int64)
    out = np.empty((m, n_heads * head_dim), dtype=np.float32)
    vmag = np.empty((m, n_heads * head_dim), dtype=np.float64)
    smag = np.empty((m, n_heads), dtype=np.float64)
    scratch = np.empty(max(1, tmax), dtype=np.float64)
    bad = _load().orc_attention(pq, m, q.shape[1], n_heads, n_kv, head_dim, pk, pv, n_slots, tmax, ps, pp,
                                out.ctypes.data, vmag.ctypes.data, smag.ctypes.data, scratch.ctypes.data)
    return out, vmag, smag, int(bad)


def kv_append(k_cache, v_cache, k, v, slot, pos, n_kv: int, head_dim: int) -> int:
    """R21: write the rows' keys k and values v ([m][n_kv hd] fp32) rounded to
    bfloat16 into the caches (in place) at [slot][g][pos]; rows out of range are
    skipped. Returns how many were skipped."""
    n_slots, _, tmax, _ = k_cache.shape
    kb = round_bf16(np.asarray(k, dtype=np.float32)).reshape(-1, n_kv, head_dim)
    vb = round_bf16(np.asarray(v, dtype=np.float32)).reshape(-1, n_kv, head_dim)
    skipped = 0
    for r, (s, p) in enumerate(zip(np.asarray(slot).tolist(), np.asarray(pos).tolist())):
        if not (0 <= s < n_slots and 0 <= p < tmax):
            skipped += 1
            continue
        k_cache[s, :, p, :] = kb[r]
        v_cache[s, :, p, :] = vb[r]
    return skipped


def quant_absmax(x):
    """O4: per-token codes and fp32 deq."""
    x, px = _c(x, np.float32)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.int8)
    deq = np.empty(m, dtype=np.float32)
    _load().orc_quant_absmax(px, m, k, q.ctypes.data, deq.ctypes.data)
    return q, deq


def quant_rms(x, gain=None, eps: float = 1e-5):
    """O5: RMSNorm (gain, eps) folded into the per-token quantization."""
    x, px = _c(x, np.float32)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.int8)
    deq = np.empty(m, dtype=np.float32)
    v = np.empty(k, dtype=np.float32)
    pg = None
    if gain is not None:
        gain, pg = _c(gain, np.float32)
    _load().orc_quant_rms(px, m, k, pg, ctypes.c_float(eps), q.ctypes.data, deq.ctypes.data, v.ctypes.data)
    return q, deq


def relu2_mul(gu, inter: int) -> np.ndarray:
    """O6: rows [gate | up] -> relu(gate)^2 * up (fp32, left to right)."""
    gu, pg = _c(gu, np.float32)
    m = gu.shape[0]
    assert gu.shape[1] == 2 * inter
    out = np.empty((m, inter), dtype=np.float32)
    _load().orc_relu2_mul(pg, m, inter, out.ctypes.data)
    return out


def contract(q, c) -> np.ndarray:
    """O7: acc = q @ c^T exactly (int32)."""
    q, pq = _c(q, np.int8)
    c, pc = _c(c, np.int8)
    m, k = q.shape
    n = c.shape[0]
    assert c.shape[1] == k
    acc = np.empty((m, n), dtype=np.int32)
    if _load().orc_contract(pq, m, k, pc, n, acc.ctypes.data) != 0:
        raise OverflowError("contraction does not fit int32")
    return acc


def rescale(acc, deq, gammas, seg_end) -> np.ndarray:
    """O8: y = fl32(fl32(acc * deq) * fl32(gamma_seg)), no bias."""
    acc, pa = _c(acc, np.int32)
    deq, pd = _c(deq, np.float32)
    g, pg = _c(np.atleast_1d(np.asarray(gammas, dtype=np.float64)), np.float64)
    se, ps = _c(np.atleast_1d(np.asarray(seg_end, dtype=np.int64)), np.int64)
    m, n = acc.shape
    assert len(g) == len(se) and se[-1] == n
    y = np.empty((m, n), dtype=np.float32)
    _load().orc_rescale(pa, m, n, pd, pg, ps, len(g), y.ctypes.data)
    return y


# ---------------------------------------------------------------- compositions
def forward(x, c, gammas, seg_end=None, gain=None, eps: float | None = None):
    """One projection: O4 (or O5 when ``eps`` is given) -> O7 -> O8."""
    n = c.shape[0]
    if seg_end is None:
        seg_end = [n]
    if eps is None:
        q, deq = quant_absmax(x)
    else:
        q, deq = quant_rms(x, gain, eps)
    acc = contract(q, c)
    return {"q": q, "deq": deq, "acc": acc, "y": rescale(acc, deq, gammas, seg_end)}


def ffn_block(x, c_gu, gam_gu, c_down, gam_down, ffn_gain=None, eps: float = 1e-5):
    """O9: q1 = O4(x); GU = [gate|up]; Mi = relu(G)^2 U; (q2, d2) = O5(Mi); y = down."""
    inter = c_gu.shape[0] // 2
    s1 = forward(x, c_gu, list(gam_gu), [inter, 2 * inter])
    mi = relu2_mul(s1["y"], inter)
    s2 = forward(mi, c_down, [gam_down], None, ffn_gain, eps)
    return {"q1": s1["q"], "deq1": s1["deq"], "acc_gu": s1["acc"], "gu": s1["y"], "mi": mi,
            "q2": s2["q"], "deq2": s2["deq"], "acc_down": s2["acc"], "y": s2["y"]}


def gqa_broadcast(v, n_heads: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """Per-token attention output when each token attends only to itself: query
    head h returns the value of key/value head h // (n_heads // n_kv_heads)."""
    group = n_heads // n_kv_heads
    m = v.shape[0]
    out = np.empty((m, n_heads * head_dim), dtype=np.float32)
    for h in range(n_heads):
        kv = h // group
        out[:, h * head_dim:(h + 1) * head_dim] = v[:, kv * head_dim:(kv + 1) * head_dim]
    return out


def decoder_layer(x, w, eps: float = 1e-5, n_heads: int = 20, n_kv_heads: int = 5, head_dim: int = 128):
    """O10, one block's projection stack (nnterp BitNet page, "The block, in order").

    ``w`` holds ternary codes and fp64 gammas: ``qkv`` [H + 2 kv][H] (q|k|v) with
    ``g_qkv`` (3), ``o`` [H][H] with ``g_o``, ``gu`` [2I][H] (gate|up) with ``g_gu`` (2),
    ``down`` [H][I] with ``g_down``; optional RMSNorm gains ``n_in``, ``n_attn``,
    ``n_post``, ``n_ffn`` (None = 1)."""
    hdim = x.shape[1]
    kv = n_kv_heads * head_dim
    inter = w["gu"].shape[0] // 2
    s_qkv = forward(x, w["qkv"], w["g_qkv"], [hdim, hdim + kv, hdim + 2 * kv], w.get("n_in"), eps)
    v = s_qkv["y"][:, hdim + kv:hdim + 2 * kv]
    a = gqa_broadcast(v, n_heads, n_kv_heads, head_dim)
    s_o = forward(a, w["o"], [w["g_o"]], None, w.get("n_attn"), eps)
    h = (x.astype(np.float32) + s_o["y"]).astype(np.float32)
    s_gu = forward(h, w["gu"], w["g_gu"], [inter, 2 * inter], w.get("n_post"), eps)
    mi = relu2_mul(s_gu["y"], inter)
    s_d = forward(mi, w["down"], [w["g_down"]], None, w.get("n_ffn"), eps)
    x_next = (h + s_d["y"]).astype(np.float32)
    return {"qkv": s_qkv, "attn": a, "o": s_o, "h": h, "gu": s_gu, "mi": mi, "down": s_d, "x": x_next}
