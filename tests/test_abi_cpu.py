"""C-ABI checks that need no GPU: the library loads, exports every function that
include/bitlinear.h declares, and rejects bad arguments on the host (before any
HIP call) with the documented status. No call here reaches a kernel: each one
fails validation or is an m == 0 no-op."""
import ctypes
import os
import re

import pytest

from ternary_weight_bitlinear_w1_amd import bitlinear as bl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

A = 0x100000  # a 16-byte-aligned fake device address (never dereferenced: validation fails first)
MIS = A + 4   # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 11
    L = ctypes.CDLL(bl.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert bl.lib().bitlinear_abi_version() == 3
    for s in range(7):
        assert bl.status_name(s)
    assert bl.status_name(0) == "ok"


def _fw(x=A, codes=None, deq=None, rowsum=None, m=4, k=64, w=A, n=32, gamma=(1.0,), seg=(32,), y=A, acc=None,
        path=0, ws=A, wsb=1 << 20):
    g = (ctypes.c_float * max(1, len(gamma)))(*gamma)
    s = (ctypes.c_int64 * max(1, len(seg)))(*seg)
    return bl.lib().bitlinear_forward(x, codes, deq, rowsum, m, k, w, n, g, s, len(gamma), y, acc, path, ws, wsb,
                                      None)


def test_forward_validation():
    assert _fw(x=None) == bl.ERR_NULL
    assert _fw(w=None) == bl.ERR_NULL
    assert _fw(y=None) == bl.ERR_NULL
    assert _fw(k=24) == bl.ERR_SHAPE
    assert _fw(k=0) == bl.ERR_SHAPE
    assert _fw(m=-1) == bl.ERR_SHAPE
    assert _fw(n=0, seg=(0,)) == bl.ERR_SHAPE
    assert _fw(seg=(31,)) == bl.ERR_SHAPE              # segments must end at n
    assert _fw(gamma=(1.0, 2.0), seg=(20, 16)) == bl.ERR_SHAPE  # not ascending
    assert _fw(gamma=(1.0,) * 5, seg=(4, 8, 12, 16, 32)) == bl.ERR_SHAPE  # too many
    assert _fw(gamma=(), seg=()) == bl.ERR_SHAPE
    assert _fw(path=7) == bl.ERR_ARG
    assert _fw(path=bl.PATH_DECODE, m=17) == bl.ERR_SHAPE
    assert _fw(x=MIS) == bl.ERR_ALIGN
    assert _fw(y=MIS) == bl.ERR_ALIGN
    assert _fw(ws=None) == bl.ERR_WORKSPACE
    assert _fw(wsb=16) == bl.ERR_WORKSPACE
    assert _fw(m=0) == bl.OK  # empty input is a no-op
    assert _fw(m=0, x=None, y=None, ws=None) == bl.OK
    assert b"seg_end" in bl.lib().bitlinear_last_error() or True


def test_forward_workspace_sizes():
    f = bl.lib().bitlinear_forward_workspace_bytes
    assert f(4, 32, 64, 0) >= 16
    assert f(4, 32, 64, 1) >= 4 * 64 + 16 + 16
    assert f(4096, 13824, 2560, 1) >= 4096 * 2560


def test_forward_workspace_holds_split_partials():
    """Few output tiles: K is split and the workspace holds the int32 partial
    sums (at least two ranges of m x n)."""
    f = bl.lib().bitlinear_forward_workspace_bytes
    assert f(64, 2560, 6912, 0) >= 2 * 64 * 2560 * 4
    assert f(4096, 2560, 6912, 0) < 4096 * 2560 * 4  # many tiles: no split


def _glu(x=A, codes=None, deq=None, rowsum=None, m=4, k=64, w=A, inter=32, gamma=(1.0, 2.0), y=A, path=0, ws=A,
         wsb=1 << 20):
    g = (ctypes.c_float * 2)(*gamma)
    return bl.lib().bitlinear_forward_relu2_glu(x, codes, deq, rowsum, m, k, w, inter, g, y, path, ws, wsb, None)


def test_forward_relu2_glu_validation():
    L = bl.lib()
    assert L.bitlinear_forward_relu2_glu(A, None, None, None, 4, 64, A, 32, None, A, 0, A, 1 << 20, None) == bl.ERR_NULL
    assert _glu(x=None) == bl.ERR_NULL
    assert _glu(w=None) == bl.ERR_NULL
    assert _glu(y=None) == bl.ERR_NULL
    assert _glu(inter=0) == bl.ERR_SHAPE
    assert _glu(inter=30) == bl.ERR_SHAPE  # inter % 4
    assert _glu(k=24) == bl.ERR_SHAPE
    assert _glu(m=-1) == bl.ERR_SHAPE
    assert _glu(path=9) == bl.ERR_ARG
    assert _glu(path=bl.PATH_DECODE, m=17) == bl.ERR_SHAPE
    assert _glu(x=MIS) == bl.ERR_ALIGN
    assert _glu(y=MIS) == bl.ERR_ALIGN
    assert _glu(ws=None) == bl.ERR_WORKSPACE
    assert _glu(m=0) == bl.OK
    assert _glu(m=0, x=None, y=None, ws=None) == bl.OK


def test_forward_relu2_glu_workspace_sizes():
    f = bl.lib().bitlinear_forward_relu2_glu_workspace_bytes
    # fused gating (m > 64, k % 128 == 0, inter % 128 == 0): no room for gate|up
    assert f(4096, 6912, 2560, 0, bl.PATH_AUTO) < 4096 * 2 * 6912 * 4
    # decode path: gate|up goes through the workspace
    assert f(4, 6912, 2560, 0, bl.PATH_AUTO) >= 4 * 2 * 6912 * 4
    assert f(4096, 6912, 2560, 0, bl.PATH_DECODE) >= 4096 * 2 * 6912 * 4


def _onl(x=A, codes=None, deq=None, rowsum=None, m=4, k=64, w=A, n=32, seg=(32,), gamma=None, y=A, acc=None, path=0,
         ws=A, wsb=1 << 24, dtype=bl.MASTER_F32):
    s = (ctypes.c_int64 * max(1, len(seg)))(*seg)
    return bl.lib().bitlinear_forward_online(x, codes, deq, rowsum, m, k, w, dtype, n, s if seg else None, len(seg),
                                             gamma, y, acc, path, ws, wsb, None)


def test_forward_online_validation():
    assert _onl(w=None) == bl.ERR_NULL
    assert _onl(x=None) == bl.ERR_NULL
    assert _onl(y=None) == bl.ERR_NULL
    assert _onl(seg=()) == bl.ERR_NULL     # seg_end is required
    assert _onl(seg=(31,)) == bl.ERR_SHAPE
    assert _onl(seg=(20, 10)) == bl.ERR_SHAPE
    assert _onl(k=24) == bl.ERR_SHAPE
    assert _onl(path=5) == bl.ERR_ARG
    assert _onl(w=MIS) == bl.ERR_ALIGN
    assert _onl(dtype=2) == bl.ERR_ARG
    assert _onl(dtype=bl.MASTER_BF16, w=MIS) == bl.ERR_ALIGN
    assert _onl(ws=None) == bl.ERR_WORKSPACE
    assert _onl(wsb=64) == bl.ERR_WORKSPACE


def test_forward_online_workspace_sizes():
    f = bl.lib().bitlinear_forward_online_workspace_bytes
    seg = (ctypes.c_int64 * 2)(6912, 13824)
    # the packed copy of the masters and the forward's own workspace
    assert f(1, 13824, 2560, 1, seg, 2) >= 13824 * 2560 // 4 + bl.lib().bitlinear_forward_workspace_bytes(1, 13824,
                                                                                                           2560, 1)
    assert f(1, 13824, 2560, 1, None, 2) == 0


def _b3(x=A, codes=None, deq=None, m=4, k=64, w=A, n=32, gamma=(1.0,), seg=(32,), y=A, acc=None, ws=A,
        wsb=1 << 20):
    g = (ctypes.c_float * max(1, len(gamma)))(*gamma)
    s = (ctypes.c_int64 * max(1, len(seg)))(*seg)
    return bl.lib().bitlinear_forward_base3(x, codes, deq, m, k, w, n, g, s, len(gamma), y, acc, ws, wsb, None)


def test_base3_row_bytes():
    f = bl.lib().bitlinear_base3_row_bytes
    assert [f(k) for k in (16, 80, 96, 2560, 6912, 8192)] == [16, 16, 32, 512, 1392, 1648]
    assert f(0) == 0


def test_forward_base3_validation():
    assert _b3(x=None) == bl.ERR_NULL
    assert _b3(w=None) == bl.ERR_NULL
    assert _b3(y=None) == bl.ERR_NULL
    assert _b3(m=5) == bl.ERR_SHAPE       # one to four tokens
    assert _b3(k=8208) == bl.ERR_SHAPE    # k <= 8192
    assert _b3(k=24) == bl.ERR_SHAPE      # k % 16
    assert _b3(m=-1) == bl.ERR_SHAPE
    assert _b3(seg=(31,)) == bl.ERR_SHAPE
    assert _b3(w=MIS) == bl.ERR_ALIGN
    assert _b3(ws=None) == bl.ERR_WORKSPACE  # x given: the codes need room
    assert _b3(wsb=16) == bl.ERR_WORKSPACE
    assert _b3(m=0) == bl.OK


def test_forward_base3_workspace_sizes():
    f = bl.lib().bitlinear_forward_base3_workspace_bytes
    assert f(4, 2560, 0) == 0
    assert f(4, 2560, 1) >= 4 * 2560 + 16 + 16
    assert f(0, 2560, 1) == 0


def test_pack_base3_validation():
    p = bl.lib().bitlinear_pack_base3
    assert p(None, 32, 64, A, None) == bl.ERR_NULL
    assert p(A, 32, 64, None, None) == bl.ERR_NULL
    assert p(A, 0, 64, A, None) == bl.ERR_SHAPE
    assert p(A, 32, 24, A, None) == bl.ERR_SHAPE
    assert p(MIS, 32, 64, A, None) == bl.ERR_ALIGN
    assert p(A, 32, 64, MIS, None) == bl.ERR_ALIGN


def test_embed_and_lm_head_validation():
    L = bl.lib()
    assert L.bitlinear_embed(None, 4, A, 100, 64, A, None) == bl.ERR_NULL
    assert L.bitlinear_embed(A, -1, A, 100, 64, A, None) == bl.ERR_SHAPE
    assert L.bitlinear_embed(A, 4, A, 0, 64, A, None) == bl.ERR_SHAPE
    assert L.bitlinear_embed(A, 4, A, 100, 60, A, None) == bl.ERR_SHAPE     # k % 8 != 0
    assert L.bitlinear_embed(A, 4, A, 100, 4104, A, None) == bl.ERR_SHAPE   # k > 4096
    assert L.bitlinear_embed(A, 4, MIS, 100, 64, A, None) == bl.ERR_ALIGN
    assert L.bitlinear_embed(None, 0, None, 100, 64, None, None) == bl.OK

    def head(x=A, m=4, k=2560, gain=None, eps=1e-5, w=A, n=1000, y=A, normed=None, ws=A, wsb=1 << 20):
        return L.bitlinear_lm_head(x, m, k, gain, eps, w, n, y, normed, ws, wsb, None)

    assert head(x=None) == bl.ERR_NULL
    assert head(w=None) == bl.ERR_NULL
    assert head(y=None) == bl.ERR_NULL
    assert head(k=2564) == bl.ERR_SHAPE     # k % 8
    assert head(k=4104) == bl.ERR_SHAPE     # k <= 4096
    assert head(n=0) == bl.ERR_SHAPE
    assert head(eps=-1.0) == bl.ERR_ARG
    assert head(w=MIS) == bl.ERR_ALIGN
    assert head(ws=None) == bl.ERR_WORKSPACE
    assert head(wsb=16) == bl.ERR_WORKSPACE
    assert head(m=0) == bl.OK
    assert L.bitlinear_lm_head_workspace_bytes(4, 2560) >= 4 * 2560 * 2
    assert L.bitlinear_lm_head_workspace_bytes(0, 2560) == 0


def test_rope_cache_attention_validation():
    L = bl.lib()
    assert L.bitlinear_rope(None, 4, 3840, 0, 20, 128, A, A, 4096, None) == bl.ERR_NULL
    assert L.bitlinear_rope(A, 4, 3840, 0, 20, 128, A, None, 4096, None) == bl.ERR_NULL  # no table
    assert L.bitlinear_rope(A, 4, 3840, 0, 20, 127, A, A, 4096, None) == bl.ERR_SHAPE   # odd head_dim
    assert L.bitlinear_rope(A, 4, 2560, 128, 20, 128, A, A, 4096, None) == bl.ERR_SHAPE  # past the row
    assert L.bitlinear_rope(A, 4, 3840, 0, 20, 128, A, A, 0, None) == bl.ERR_SHAPE     # empty table
    assert L.bitlinear_rope(A, 4, 3840, 0, 20, 128, A, A + 4, 4096, None) == bl.ERR_ALIGN
    assert L.bitlinear_rope(None, 0, 3840, 0, 20, 128, None, None, 4096, None) == bl.OK
    tab = (ctypes.c_float * 8)()
    assert L.bitlinear_rope_table(5e5, 8, 1, None) == bl.ERR_NULL
    assert L.bitlinear_rope_table(5e5, 7, 1, tab) == bl.ERR_SHAPE
    assert L.bitlinear_rope_table(5e5, 8, 0, tab) == bl.ERR_SHAPE
    assert L.bitlinear_rope_table(0.0, 8, 1, tab) == bl.ERR_ARG
    assert L.bitlinear_rope_table(float("inf"), 8, 1, tab) == bl.ERR_ARG
    app = L.bitlinear_kv_append
    assert app(A, A, 4, 3840, 5, 128, None, A, A, A, 8, 4096, None) == bl.ERR_NULL
    assert app(A, A, 4, 600, 5, 128, A, A, A, A, 8, 4096, None) == bl.ERR_SHAPE     # 640 > ld
    assert app(A, A, 4, 3840, 5, 128, A, A, A, A, 0, 4096, None) == bl.ERR_SHAPE
    att = L.bitlinear_attention_decode

    def call(m=4, ldq=3840, nh=20, nkv=5, hd=128, ws=A, wsb=1 << 30, q=A):
        return att(q, m, ldq, nh, nkv, hd, A, A, 8, 4096, A, A, A, 2560, ws, wsb, None)

    assert call(q=None) == bl.ERR_NULL
    assert call(hd=64) == bl.ERR_SHAPE        # head_dim 128 only
    assert call(nh=21) == bl.ERR_SHAPE        # heads % kv heads
    assert call(nh=40) == bl.ERR_SHAPE        # at most 8 query heads per kv head
    assert call(ldq=2000) == bl.ERR_SHAPE
    assert call(ws=None) == bl.ERR_WORKSPACE
    assert call(m=0) == bl.OK
    assert L.bitlinear_attention_workspace_bytes(4, 20, 4096) >= 4 * 20 * 16 * 130 * 4


def test_quantize_acts_validation():
    q = bl.lib().bitlinear_quantize_acts
    assert q(None, 4, 64, 0, None, ctypes.c_float(1e-5), A, A, None, None) == bl.ERR_NULL
    assert q(A, 4, 60, 0, None, ctypes.c_float(1e-5), A, A, None, None) == bl.ERR_SHAPE
    assert q(A, 4, 64, 9, None, ctypes.c_float(1e-5), A, A, None, None) == bl.ERR_ARG
    assert q(MIS, 4, 64, 0, None, ctypes.c_float(1e-5), A, A, None, None) == bl.ERR_ALIGN
    assert q(A, 4, 64, 1, MIS, ctypes.c_float(1e-5), A, A, None, None) == bl.ERR_ALIGN
    assert q(A, 0, 64, 0, None, ctypes.c_float(1e-5), A, A, None, None) == bl.OK
    # m == 0: the per-token buffers may be NULL (an empty tensor's data pointer)
    assert q(None, 0, 64, 0, None, ctypes.c_float(1e-5), None, None, None, None) == bl.OK


def test_quantize_weights_validation():
    f = bl.lib().bitlinear_quantize_weights
    assert f(None, 8, 64, None, A, A, A, 1 << 20, None) == bl.ERR_NULL
    assert f(A, 8, 64, None, A, None, A, 1 << 20, None) == bl.ERR_NULL
    assert f(A, 8, 40, None, A, A, A, 1 << 20, None) == bl.ERR_SHAPE
    assert f(A, -1, 64, None, A, A, A, 1 << 20, None) == bl.ERR_SHAPE
    assert f(A, 8, 64, None, MIS, A, A, 1 << 20, None) == bl.ERR_ALIGN
    assert f(A, 8, 64, None, A, A, None, 0, None) == bl.ERR_WORKSPACE
    assert bl.lib().bitlinear_quantize_weights_workspace_bytes(13824, 2560) >= 8
    v = bl.lib().bitlinear_validate_packed
    assert v(None, 8, 64, A, None) == bl.ERR_NULL
    assert v(A, 8, 20, A, None) == bl.ERR_SHAPE


def _block(kind=bl.BLOCK_DECODER, H=64, I=96, nh=8, nkv=2, hd=8, layers=1, null_w=False):
    arr = (bl.Layer * layers)()
    for i in range(layers):
        arr[i].qkv = None if null_w else A
        arr[i].o = A
        arr[i].gate_up = A
        arr[i].down = A
    return bl.Block(kind, layers, H, I, nh, nkv, hd, 1e-5, arr), arr


def test_large_shapes_leave_the_32bit_pipelined_gemm():
    """Codes or packed weights of 2^31 bytes and more take the generic GEMM
    (64-bit offsets), which does not split K: no partial-sum workspace."""
    f = bl.lib().bitlinear_forward_workspace_bytes
    k_under, k_over = (1 << 25) - 128, 1 << 25  # 256 rows of k/4 bytes: under / at 2^31
    assert f(64, 256, k_under, 0) > 256       # the pipelined 64-token tile splits K
    assert f(64, 256, k_over, 0) == 256       # row sums only


def test_block_validation():
    f = bl.lib().bitlinear_block_forward
    blk, keep = _block()
    assert bl.lib().bitlinear_block_workspace_bytes(ctypes.byref(blk), 4) > 0
    assert f(ctypes.byref(blk), A, 0, A, None, None, 0, None) == bl.OK  # m == 0
    assert f(ctypes.byref(blk), None, 0, None, None, None, 0, None) == bl.OK
    assert f(ctypes.byref(blk), None, 4, A, None, None, 0, None) == bl.ERR_NULL
    assert f(ctypes.byref(blk), A, 4, A, None, None, 0, None) == bl.ERR_WORKSPACE
    assert f(ctypes.byref(blk), None, 4, A, None, A, 1 << 30, None) == bl.ERR_NULL
    assert f(ctypes.byref(blk), MIS, 4, A, None, A, 1 << 30, None) == bl.ERR_ALIGN
    bad, k1 = _block(kind=5)
    assert f(ctypes.byref(bad), A, 4, A, None, A, 1 << 30, None) == bl.ERR_ARG
    bad, k2 = _block(nh=6)  # 6 * 8 != 64
    assert f(ctypes.byref(bad), A, 4, A, None, A, 1 << 30, None) == bl.ERR_SHAPE
    bad, k3 = _block(nh=8, nkv=3)  # 3 does not divide 8
    assert f(ctypes.byref(bad), A, 4, A, None, A, 1 << 30, None) == bl.ERR_SHAPE
    bad, k4 = _block(null_w=True)
    assert f(ctypes.byref(bad), A, 4, A, None, A, 1 << 30, None) == bl.ERR_NULL
    bad, k5 = _block(kind=bl.BLOCK_FFN, layers=2)
    assert f(ctypes.byref(bad), A, 4, A, None, A, 1 << 30, None) == bl.ERR_SHAPE
    bad, k6 = _block(H=72)
    assert f(ctypes.byref(bad), A, 4, A, None, A, 1 << 30, None) == bl.ERR_SHAPE
    assert f(None, A, 4, A, None, A, 1 << 30, None) == bl.ERR_NULL


def test_cached_block_needs_a_rope_table():
    f = bl.lib().bitlinear_block_forward
    blk, keep = _block(kind=bl.BLOCK_DECODER_CACHED, H=256, I=96, nh=2, nkv=1, hd=128)
    for i in range(1):
        keep[i].k_cache = keep[i].v_cache = A
    blk.slot = blk.pos = A
    blk.n_slots, blk.t_max = 2, 64
    assert f(ctypes.byref(blk), A, 4, A, None, A, 1 << 30, None) == bl.ERR_NULL  # no table
    blk.rope_table, blk.rope_n_pos = A + 4, 4096
    assert f(ctypes.byref(blk), A, 4, A, None, A, 1 << 30, None) == bl.ERR_ALIGN
    blk.rope_table, blk.rope_n_pos = A, 0
    assert f(ctypes.byref(blk), A, 4, A, None, A, 1 << 30, None) == bl.ERR_SHAPE


def test_rope_table_equals_the_oracle_angles():
    """The host-built rotary table ([nnterp] "Loading": theta 500,000, 4096
    positions) holds, bit for bit, the fp32 cosines and sines the oracle rotates
    with: rotating the unit vector on the first element of each pair gives (c, s)."""
    import numpy as np
    import oracle
    hd, n_pos = 128, 4096
    tab = np.empty((n_pos, hd // 2, 2), dtype=np.float32)
    assert bl.lib().bitlinear_rope_table(5e5, hd, n_pos, tab.ctypes.data) == bl.OK
    x = np.zeros((n_pos, hd), dtype=np.float32)
    x[:, :hd // 2] = 1.0
    ref = oracle.rope(x, np.arange(n_pos), 1, hd, 5e5, n_pos=n_pos)
    assert np.array_equal(tab[:, :, 0].view(np.uint32), ref[:, :hd // 2].view(np.uint32))
    assert np.array_equal(tab[:, :, 1].view(np.uint32), ref[:, hd // 2:].view(np.uint32))
    assert np.all(tab[0, :, 0] == 1.0) and np.all(tab[0, :, 1] == 0.0)


def test_library_refuses_to_load_when_missing(tmp_path, monkeypatch):
    """The binding has no fallback: with the library path pointing nowhere it raises."""
    monkeypatch.setattr(bl, "_lib", None)
    monkeypatch.setattr(bl, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        bl.lib()


def test_probe_validation():
    L = bl.lib()
    for probe in (L.bitlinear_probe_mfma, L.bitlinear_probe_mfma_varied):
        assert probe(10, 4, None, None) == bl.ERR_NULL
        assert probe(0, 4, A, None) == bl.ERR_SHAPE
        assert probe(10, 0, A, None) == bl.ERR_SHAPE
        assert probe(10, 65537, A, None) == bl.ERR_SHAPE
    assert L.bitlinear_probe_read(A, 0, 0, A, None) == bl.OK  # nothing to read: a no-op
    assert L.bitlinear_probe_read(None, 64, 0, A, None) == bl.ERR_NULL
    assert L.bitlinear_probe_read(A, 24, 0, A, None) == bl.ERR_SHAPE
    assert L.bitlinear_probe_read(MIS, 64, 0, A, None) == bl.ERR_ALIGN
