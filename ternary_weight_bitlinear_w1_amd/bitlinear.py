"""Python binding of the gfx950 BitLinear library (``libbitlinear.so``).

Argument marshalling only: every function below checks nothing the library
does not check itself, takes torch tensors for device memory, passes their
device pointers and the current HIP stream to the C entry point of the same
name (``include/bitlinear.h``) and raises :class:`BitLinearError` on a non-OK
status. All arithmetic runs in the HIP kernels; if the library is not built,
loading fails with an error (there is no other implementation to fall back to).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_DEVICE, ERR_ARG = range(7)
ACT_ABSMAX, ACT_RMSNORM, ACT_RELU2_RMSNORM = 0, 1, 2
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2
BLOCK_FFN, BLOCK_DECODER, BLOCK_DECODER_CACHED = 0, 1, 2
MASTER_F32, MASTER_BF16 = 0, 1
MAX_SEGMENTS = 4

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class BitLinearError(RuntimeError):
    def __init__(self, func: str, status: int, detail: str):
        super().__init__(f"{func}: {status_name(status)} ({detail})")
        self.status = status


class Layer(ctypes.Structure):
    _fields_ = [("qkv", _p), ("qkv_gamma", ctypes.c_float * 3), ("o", _p), ("o_gamma", ctypes.c_float),
                ("gate_up", _p), ("gate_up_gamma", ctypes.c_float * 2), ("down", _p), ("down_gamma", ctypes.c_float),
                ("input_norm_gain", _p), ("attn_sub_norm_gain", _p), ("post_attn_norm_gain", _p),
                ("ffn_sub_norm_gain", _p), ("k_cache", _p), ("v_cache", _p)]


class Block(ctypes.Structure):
    _fields_ = [("kind", _i32), ("n_layers", _i32), ("hidden", _i64), ("intermediate", _i64),
                ("n_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32), ("eps", ctypes.c_float),
                ("layers", ctypes.POINTER(Layer)), ("slot", _p), ("pos", _p), ("n_slots", _i64), ("t_max", _i64),
                ("rope_table", _p), ("rope_n_pos", _i64)]


class Trace(ctypes.Structure):
    _fields_ = [(name, _p) for name in ("codes_in", "codes_attn", "codes_post", "codes_ffn", "deq", "qkv", "h",
                                        "gate_up", "x_out", "acc_qkv", "acc_o", "acc_gate_up", "acc_down",
                                        "attn")]


_lib = None


def lib():
    """The loaded C library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -m ternary_weight_bitlinear_w1_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "bitlinear_quantize_weights": (_i32, [_p, _i64, _i64, _p, _p, _p, _p, _sz, _p]),
            "bitlinear_quantize_weights_workspace_bytes": (_sz, [_i64, _i64]),
            "bitlinear_validate_packed": (_i32, [_p, _i64, _i64, _p, _p]),
            "bitlinear_quantize_acts": (_i32, [_p, _i64, _i64, _i32, _p, ctypes.c_float, _p, _p, _p, _p]),
            "bitlinear_forward": (_i32, [_p, _p, _p, _p, _i64, _i64, _p, _i64, _p, _p, _i32, _p, _p, _i32, _p, _sz,
                                         _p]),
            "bitlinear_forward_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
            "bitlinear_forward_noalloc": (_i32, [_p, _p, _p, _p, _i64, _i64, _p, _i64, _p, _p, _i32, _p, _p, _i32,
                                                 _p]),
            "bitlinear_forward_noalloc_max_scratch_bytes": (_sz, []),
            "bitlinear_forward_relu2_glu": (_i32, [_p, _p, _p, _p, _i64, _i64, _p, _i64, _p, _p, _i32, _p, _sz, _p]),
            "bitlinear_forward_online": (_i32, [_p, _p, _p, _p, _i64, _i64, _p, _i32, _i64, _p, _i32, _p, _p, _p, _i32,
                                                _p, _sz, _p]),
            "bitlinear_forward_online_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _p, _i32]),
            "bitlinear_forward_relu2_glu_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32]),
            "bitlinear_embed": (_i32, [_p, _i64, _p, _i64, _i64, _p, _p]),
            "bitlinear_lm_head": (_i32, [_p, _i64, _i64, _p, ctypes.c_float, _p, _i64, _p, _p, _p, _sz, _p]),
            "bitlinear_lm_head_workspace_bytes": (_sz, [_i64, _i64]),
            "bitlinear_rope_table": (_i32, [ctypes.c_double, _i32, _i64, _p]),
            "bitlinear_rope": (_i32, [_p, _i64, _i64, _i64, _i32, _i32, _p, _p, _i64, _p]),
            "bitlinear_kv_append": (_i32, [_p, _p, _i64, _i64, _i32, _i32, _p, _p, _p, _p, _i64, _i64, _p]),
            "bitlinear_attention_decode": (_i32, [_p, _i64, _i64, _i32, _i32, _i32, _p, _p, _i64, _i64, _p, _p, _p,
                                                  _i64, _p, _sz, _p]),
            "bitlinear_attention_workspace_bytes": (_sz, [_i64, _i32, _i64]),
            "bitlinear_base3_row_bytes": (_sz, [_i64]),
            "bitlinear_pack_base3": (_i32, [_p, _i64, _i64, _p, _p]),
            "bitlinear_forward_base3": (_i32, [_p, _p, _p, _i64, _i64, _p, _i64, _p, _p, _i32, _p, _p, _p, _sz, _p]),
            "bitlinear_forward_base3_workspace_bytes": (_sz, [_i64, _i64, _i32]),
            "bitlinear_block_forward": (_i32, [ctypes.POINTER(Block), _p, _i64, _p, ctypes.POINTER(Trace), _p, _sz,
                                               _p]),
            "bitlinear_block_workspace_bytes": (_sz, [ctypes.POINTER(Block), _i64]),
            "bitlinear_probe_read": (_i32, [_p, _i64, _i64, _p, _p]),
            "bitlinear_probe_mfma": (_i32, [_i32, _i64, _p, _p]),
            "bitlinear_probe_mfma_varied": (_i32, [_i32, _i64, _p, _p]),
            "bitlinear_status_str": (ctypes.c_char_p, [_i32]),
            "bitlinear_last_error": (ctypes.c_char_p, []),
            "bitlinear_abi_version": (_i32, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_name(status: int) -> str:
    return lib().bitlinear_status_str(status).decode()


def _check(func: str, status: int) -> None:
    if status != OK:
        raise BitLinearError(func, status, lib().bitlinear_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device):
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device) if nbytes else None


# ---------------------------------------------------------------------------------------------
def quantize_weights(w: torch.Tensor, gamma_in: Optional[torch.Tensor] = None):
    """Absmean-ternarize and pack ``w`` [n][k] fp32 -> (packed [n][k/4] uint8, gamma [1] fp64)."""
    n, k = w.shape
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device=w.device)
    gamma = torch.empty(1, dtype=torch.float64, device=w.device)
    nb = lib().bitlinear_quantize_weights_workspace_bytes(n, k)
    ws = _workspace(nb, w.device)
    _check("bitlinear_quantize_weights",
           lib().bitlinear_quantize_weights(_ptr(w), n, k, _ptr(gamma_in), _ptr(packed), _ptr(gamma), _ptr(ws),
                                            nb, _stream(w.device)))
    return packed, gamma


def validate_packed(packed: torch.Tensor, k: int) -> int:
    """Number of invalid (== 3) fields in a packed matrix (synchronizes)."""
    out = torch.empty(1, dtype=torch.int64, device=packed.device)
    _check("bitlinear_validate_packed",
           lib().bitlinear_validate_packed(_ptr(packed), packed.shape[0], k, _ptr(out), _stream(packed.device)))
    return int(out.item())


def quantize_acts(x: torch.Tensor, mode: int = ACT_ABSMAX, gain: Optional[torch.Tensor] = None, eps: float = 1e-5):
    """Per-token int8 codes of ``x`` -> (codes [m][k] int8, deq [m] fp32, rowsum [m] int32).
    For ACT_RELU2_RMSNORM, ``x`` is [m][2k] ([gate | up] rows)."""
    m, kk = x.shape
    k = kk // 2 if mode == ACT_RELU2_RMSNORM else kk
    codes = torch.empty((m, k), dtype=torch.int8, device=x.device)
    deq = torch.empty(m, dtype=torch.float32, device=x.device)
    rowsum = torch.empty(m, dtype=torch.int32, device=x.device)
    _check("bitlinear_quantize_acts",
           lib().bitlinear_quantize_acts(_ptr(x), m, k, mode, _ptr(gain), ctypes.c_float(eps), _ptr(codes),
                                         _ptr(deq), _ptr(rowsum), _stream(x.device)))
    return codes, deq, rowsum


def forward(packed: torch.Tensor, k: int, gamma: Sequence[float], seg_end: Optional[Sequence[int]] = None,
            x: Optional[torch.Tensor] = None, codes: Optional[torch.Tensor] = None,
            deq: Optional[torch.Tensor] = None, rowsum: Optional[torch.Tensor] = None,
            want_acc: bool = False, path: int = PATH_AUTO, out: Optional[torch.Tensor] = None):
    """One projection -> y [m][n] fp32 (and the exact int32 acc when ``want_acc``)."""
    n = packed.shape[0]
    src = x if x is not None else codes
    m = src.shape[0]
    dev = packed.device
    if seg_end is None:
        seg_end = [n]
    g = (ctypes.c_float * len(gamma))(*[float(v) for v in gamma])
    se = (ctypes.c_int64 * len(seg_end))(*[int(v) for v in seg_end])
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
    nb = lib().bitlinear_forward_workspace_bytes(m, n, k, 1 if x is not None else 0)
    ws = _workspace(nb, dev)
    _check("bitlinear_forward",
           lib().bitlinear_forward(_ptr(x), _ptr(codes), _ptr(deq), _ptr(rowsum), m, k, _ptr(packed), n, g, se,
                                   len(gamma), _ptr(y), _ptr(acc), path, _ptr(ws), nb, _stream(dev)))
    return (y, acc) if want_acc else y


def forward_noalloc(packed: torch.Tensor, k: int, gamma: Sequence[float], seg_end: Optional[Sequence[int]] = None,
                    x: Optional[torch.Tensor] = None, codes: Optional[torch.Tensor] = None,
                    deq: Optional[torch.Tensor] = None, rowsum: Optional[torch.Tensor] = None,
                    want_acc: bool = False, path: int = PATH_AUTO, out: Optional[torch.Tensor] = None,
                    acc_out: Optional[torch.Tensor] = None):
    """:func:`forward` through the entry point that allocates nothing (its
    scratch is the library's own per-device array). With ``out`` (and
    ``acc_out``) given, this function allocates nothing either."""
    n = packed.shape[0]
    src = x if x is not None else codes
    m = src.shape[0]
    dev = packed.device
    if seg_end is None:
        seg_end = [n]
    g = (ctypes.c_float * len(gamma))(*[float(v) for v in gamma])
    se = (ctypes.c_int64 * len(seg_end))(*[int(v) for v in seg_end])
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=dev)
    acc = acc_out if acc_out is not None else (
        torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None)
    _check("bitlinear_forward_noalloc",
           lib().bitlinear_forward_noalloc(_ptr(x), _ptr(codes), _ptr(deq), _ptr(rowsum), m, k, _ptr(packed), n, g,
                                           se, len(gamma), _ptr(y), _ptr(acc), path, _stream(dev)))
    return (y, acc) if acc is not None else y


def forward_online(w_master: torch.Tensor, seg_end: Optional[Sequence[int]] = None,
                   x: Optional[torch.Tensor] = None, codes: Optional[torch.Tensor] = None,
                   deq: Optional[torch.Tensor] = None, rowsum: Optional[torch.Tensor] = None,
                   want_acc: bool = False, path: int = PATH_AUTO, out: Optional[torch.Tensor] = None):
    """Online mode: ternarize the masters [n][k] (fp32, or bfloat16 given as a
    torch.bfloat16 or uint16 tensor; one gamma per segment) and project. Returns
    (y, gamma) or (y, acc, gamma); gamma is a device fp64 tensor."""
    n, k = w_master.shape
    if w_master.dtype not in (torch.float32, torch.bfloat16, torch.uint16):
        raise TypeError("forward_online takes fp32 or bfloat16 masters")
    src = x if x is not None else codes
    m = src.shape[0]
    dev = w_master.device
    if seg_end is None:
        seg_end = [n]
    se = (ctypes.c_int64 * len(seg_end))(*[int(v) for v in seg_end])
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
    gamma = torch.empty(len(seg_end), dtype=torch.float64, device=dev)
    nb = lib().bitlinear_forward_online_workspace_bytes(m, n, k, 1 if x is not None else 0, se, len(seg_end))
    ws = _workspace(nb, dev)
    _check("bitlinear_forward_online",
           lib().bitlinear_forward_online(_ptr(x), _ptr(codes), _ptr(deq), _ptr(rowsum), m, k, _ptr(w_master),
                                          MASTER_F32 if w_master.dtype == torch.float32 else MASTER_BF16, n, se,
                                          len(seg_end), _ptr(gamma), _ptr(y), _ptr(acc), path, _ptr(ws), nb,
                                          _stream(dev)))
    return (y, acc, gamma) if want_acc else (y, gamma)


def forward_relu2_glu(packed: torch.Tensor, k: int, gamma: Sequence[float], x: Optional[torch.Tensor] = None,
                      codes: Optional[torch.Tensor] = None, deq: Optional[torch.Tensor] = None,
                      rowsum: Optional[torch.Tensor] = None, path: int = PATH_AUTO,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gate and up projections with the squared-ReLU gating -> [m][inter] fp32.
    ``packed`` is [gate; up] ([2 inter][k/4]); ``gamma`` = (gate, up)."""
    inter = packed.shape[0] // 2
    src = x if x is not None else codes
    m = src.shape[0]
    dev = packed.device
    g = (ctypes.c_float * 2)(*[float(v) for v in gamma])
    y = out if out is not None else torch.empty((m, inter), dtype=torch.float32, device=dev)
    nb = lib().bitlinear_forward_relu2_glu_workspace_bytes(m, inter, k, 1 if x is not None else 0, path)
    ws = _workspace(nb, dev)
    _check("bitlinear_forward_relu2_glu",
           lib().bitlinear_forward_relu2_glu(_ptr(x), _ptr(codes), _ptr(deq), _ptr(rowsum), m, k, _ptr(packed), inter,
                                             g, _ptr(y), path, _ptr(ws), nb, _stream(dev)))
    return y


def embed(ids: torch.Tensor, table: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows of the bfloat16 table (uint16 bits [vocab][k]) for int64 ids [m] -> fp32 [m][k]."""
    vocab, k = table.shape
    m = ids.shape[0]
    x = out if out is not None else torch.empty((m, k), dtype=torch.float32, device=table.device)
    _check("bitlinear_embed", lib().bitlinear_embed(_ptr(ids), m, _ptr(table), vocab, k, _ptr(x),
                                                    _stream(table.device)))
    return x


def lm_head(x: torch.Tensor, w_head: torch.Tensor, gain: Optional[torch.Tensor] = None, eps: float = 1e-5,
            want_normed: bool = False, out: Optional[torch.Tensor] = None):
    """Final norm + bfloat16 head: x [m][k] fp32, w_head uint16 bits [vocab][k] ->
    logits [m][vocab] fp32 (and the normed bfloat16 input when ``want_normed``)."""
    m, k = x.shape
    n = w_head.shape[0]
    dev = x.device
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=dev)
    normed = torch.empty((m, k), dtype=torch.uint16, device=dev) if want_normed else None
    nb = 0 if want_normed else lib().bitlinear_lm_head_workspace_bytes(m, k)
    ws = _workspace(nb, dev)
    _check("bitlinear_lm_head",
           lib().bitlinear_lm_head(_ptr(x), m, k, _ptr(gain), eps, _ptr(w_head), n, _ptr(y), _ptr(normed), _ptr(ws),
                                   nb, _stream(dev)))
    return (y, normed) if want_normed else y


def rope_table(theta: float, head_dim: int, n_pos: int, device) -> torch.Tensor:
    """The rotary table [n_pos][head_dim/2][2] fp32, formed by the library on the
    host and copied to ``device``."""
    host = torch.empty((n_pos, head_dim // 2, 2), dtype=torch.float32)
    _check("bitlinear_rope_table", lib().bitlinear_rope_table(theta, head_dim, n_pos, host.data_ptr()))
    return host.to(device)


def rope(x: torch.Tensor, pos: torch.Tensor, n_heads: int, head_dim: int, table: torch.Tensor, col0: int = 0):
    """RoPE in place on the heads of x [m][ld] fp32 starting at column col0, with
    the rotary table from :func:`rope_table`."""
    m, ld = x.shape
    _check("bitlinear_rope", lib().bitlinear_rope(_ptr(x), m, ld, col0, n_heads, head_dim, _ptr(pos), _ptr(table),
                                                  table.shape[0], _stream(x.device)))
    return x


def kv_append(k: torch.Tensor, v: torch.Tensor, slot: torch.Tensor, pos: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor) -> None:
    """Write rows of k, v ([m][n_kv hd] fp32 views with a common row stride) into
    the bfloat16 caches [n_slots][n_kv][t_max][hd] at (slot, pos)."""
    n_slots, n_kv, t_max, hd = k_cache.shape
    m = k.shape[0]
    assert k.stride(0) == v.stride(0) and k.stride(1) == 1 and v.stride(1) == 1
    _check("bitlinear_kv_append",
           lib().bitlinear_kv_append(_ptr(k), _ptr(v), m, k.stride(0), n_kv, hd, _ptr(slot), _ptr(pos),
                                     _ptr(k_cache), _ptr(v_cache), n_slots, t_max, _stream(k.device)))


def attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, slot: torch.Tensor,
                     pos: torch.Tensor, n_heads: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Each token's causal attention over its slot's cache -> [m][n_heads hd] fp32.
    q rows hold the query heads from column 0 (any row stride)."""
    n_slots, n_kv, t_max, hd = k_cache.shape
    m = q.shape[0]
    dev = q.device
    o = out if out is not None else torch.empty((m, n_heads * hd), dtype=torch.float32, device=dev)
    nb = lib().bitlinear_attention_workspace_bytes(m, n_heads, t_max)
    ws = _workspace(nb, dev)
    _check("bitlinear_attention_decode",
           lib().bitlinear_attention_decode(_ptr(q), m, q.stride(0), n_heads, n_kv, hd, _ptr(k_cache), _ptr(v_cache),
                                            n_slots, t_max, _ptr(slot), _ptr(pos), _ptr(o), o.stride(0), _ptr(ws), nb,
                                            _stream(dev)))
    return o


def probe_read(src: torch.Tensor, nbytes: Optional[int] = None, grid: int = 0,
               sink: Optional[torch.Tensor] = None) -> None:
    """Measurement probe: read ``nbytes`` (default all) of ``src`` once."""
    nb = src.numel() * src.element_size() if nbytes is None else nbytes
    s = sink if sink is not None else torch.zeros(1, dtype=torch.int32, device=src.device)
    _check("bitlinear_probe_read", lib().bitlinear_probe_read(_ptr(src), nb, grid, _ptr(s), _stream(src.device)))


def probe_mfma(iters: int, workgroups: int, sink: torch.Tensor, varied: bool = False) -> None:
    """Measurement probe: workgroups x 4 waves x iters x 8 int8 MFMA 32x32x32,
    on fixed operands or (varied) on operands that change from one MFMA to the
    next with the value ranges of the GEMMs' operands."""
    name = "bitlinear_probe_mfma_varied" if varied else "bitlinear_probe_mfma"
    _check(name, getattr(lib(), name)(iters, workgroups, _ptr(sink), _stream(sink.device)))


def base3_row_bytes(k: int) -> int:
    """Bytes of one weight row of k codes stored five to a byte."""
    return int(lib().bitlinear_base3_row_bytes(k))


def pack_base3(packed: torch.Tensor, k: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Two-bit packed weights [n][k/4] -> the base-3 storage [n][base3_row_bytes(k)]."""
    n = packed.shape[0]
    w3 = out if out is not None else torch.empty((n, base3_row_bytes(k)), dtype=torch.uint8, device=packed.device)
    _check("bitlinear_pack_base3",
           lib().bitlinear_pack_base3(_ptr(packed), n, k, _ptr(w3), _stream(packed.device)))
    return w3


def forward_base3(w3: torch.Tensor, k: int, gamma: Sequence[float], seg_end: Optional[Sequence[int]] = None,
                  x: Optional[torch.Tensor] = None, codes: Optional[torch.Tensor] = None,
                  deq: Optional[torch.Tensor] = None, want_acc: bool = False,
                  out: Optional[torch.Tensor] = None):
    """1..4-token projection reading base-3 weights -> y [m][n] (and acc when ``want_acc``)."""
    n = w3.shape[0]
    src = x if x is not None else codes
    m = src.shape[0]
    dev = w3.device
    if seg_end is None:
        seg_end = [n]
    g = (ctypes.c_float * len(gamma))(*[float(v) for v in gamma])
    se = (ctypes.c_int64 * len(seg_end))(*[int(v) for v in seg_end])
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=dev)
    acc = torch.empty((m, n), dtype=torch.int32, device=dev) if want_acc else None
    nb = lib().bitlinear_forward_base3_workspace_bytes(m, k, 1 if x is not None else 0)
    ws = _workspace(nb, dev)
    _check("bitlinear_forward_base3",
           lib().bitlinear_forward_base3(_ptr(x), _ptr(codes), _ptr(deq), m, k, _ptr(w3), n, g, se, len(gamma),
                                         _ptr(y), _ptr(acc), _ptr(ws), nb, _stream(dev)))
    return (y, acc) if want_acc else y


# ---------------------------------------------------------------------------------------------
@dataclass
class LayerWeights:
    """Packed weights (device uint8 tensors) and fp32 scales of one block."""
    gate_up: torch.Tensor
    gate_up_gamma: Sequence[float]
    down: torch.Tensor
    down_gamma: float
    qkv: Optional[torch.Tensor] = None
    qkv_gamma: Sequence[float] = (0.0, 0.0, 0.0)
    o: Optional[torch.Tensor] = None
    o_gamma: float = 0.0
    input_norm_gain: Optional[torch.Tensor] = None
    attn_sub_norm_gain: Optional[torch.Tensor] = None
    post_attn_norm_gain: Optional[torch.Tensor] = None
    ffn_sub_norm_gain: Optional[torch.Tensor] = None
    k_cache: Optional[torch.Tensor] = None  # BLOCK_DECODER_CACHED: [n_slots][n_kv][t_max][hd] bfloat16 bits
    v_cache: Optional[torch.Tensor] = None


@dataclass
class BlockSpec:
    kind: int
    hidden: int
    intermediate: int
    layers: list = field(default_factory=list)
    n_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 0
    eps: float = 1e-5
    slot: Optional[torch.Tensor] = None   # BLOCK_DECODER_CACHED: device int64 [m]
    pos: Optional[torch.Tensor] = None
    rope_table: Optional[torch.Tensor] = None  # BLOCK_DECODER_CACHED: device [n_pos][head_dim/2][2] (rope_table())

    def to_c(self):
        arr = (Layer * len(self.layers))()
        for i, L in enumerate(self.layers):
            arr[i] = Layer(_ptr(L.qkv), (ctypes.c_float * 3)(*[float(v) for v in L.qkv_gamma]), _ptr(L.o),
                           float(L.o_gamma), _ptr(L.gate_up),
                           (ctypes.c_float * 2)(*[float(v) for v in L.gate_up_gamma]), _ptr(L.down),
                           float(L.down_gamma), _ptr(L.input_norm_gain), _ptr(L.attn_sub_norm_gain),
                           _ptr(L.post_attn_norm_gain), _ptr(L.ffn_sub_norm_gain), _ptr(L.k_cache), _ptr(L.v_cache))
        n_slots = t_max = 0
        kc = self.layers[0].k_cache if self.layers else None
        if kc is not None:
            n_slots, t_max = kc.shape[0], kc.shape[2]
        blk = Block(self.kind, len(self.layers), self.hidden, self.intermediate, self.n_heads, self.n_kv_heads,
                    self.head_dim, self.eps, arr, _ptr(self.slot), _ptr(self.pos), n_slots, t_max,
                    _ptr(self.rope_table), self.rope_table.shape[0] if self.rope_table is not None else 0)
        return blk, arr


def block_workspace_bytes(spec: BlockSpec, m: int) -> int:
    blk, _keep = spec.to_c()
    return int(lib().bitlinear_block_workspace_bytes(ctypes.byref(blk), m))


def block_forward(spec: BlockSpec, x: torch.Tensor, trace: Optional[dict] = None,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Run a block chain on x [m][H] -> y [m][H]. ``trace`` maps Trace field names to
    preallocated device tensors (see include/bitlinear.h)."""
    blk, _keep = spec.to_c()
    m = x.shape[0]
    y = out if out is not None else torch.empty_like(x)
    nb = int(lib().bitlinear_block_workspace_bytes(ctypes.byref(blk), m))
    ws = workspace if workspace is not None else _workspace(nb, x.device)
    tr = None
    if trace:
        tr = Trace(**{k: _ptr(v) for k, v in trace.items()})
    _check("bitlinear_block_forward",
           lib().bitlinear_block_forward(ctypes.byref(blk), _ptr(x), m, _ptr(y),
                                         ctypes.byref(tr) if tr is not None else None, _ptr(ws),
                                         ws.numel() if ws is not None else 0, _stream(x.device)))
    return y
