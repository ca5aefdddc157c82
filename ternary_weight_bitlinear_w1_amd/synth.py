"""Seeded synthetic inputs for the BitLinear hot path (Python side of ``synth.c``).

This module and ``synth.c`` only draw random numbers. They hold none of the
method's arithmetic (no quantisation, no contraction, no rescale), so both the
HIP path's tests and the CPU oracle take their inputs from here without sharing
any of the computation under test.

Generator (counter based, so any element can be drawn on its own):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): output ``i`` of the stream with seed ``s`` is
  ``mix(s + (i + 1) * 0x9E3779B97F4A7C15 mod 2**64)`` with the published
  finaliser ``mix``.
* A tensor's stream seed is output 0 of the stream seeded with
  ``base ^ (config << 40) ^ (layer << 16) ^ tensor`` (:func:`stream_seed`).
* Normal draws: Box-Muller in fp64 on outputs ``2i`` and ``2i + 1`` (see
  ``synth.c``); the value is ``float32(sigma * z)``.
* Outlier channels: ``n`` channels drawn without replacement by a partial
  Fisher-Yates shuffle on their own stream; the drawn fp32 value in those
  channels is multiplied by 20 in fp32 (one rounding).

Inputs are generated on the host once and copied to both sides, so parity
never depends on a device's libm.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# tensor ids (any distinct small ints work)
T_WEIGHT, T_ACT, T_OUTLIER, T_GAIN, T_ACT2 = 1, 2, 3, 4, 5


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_u64.restype = ctypes.c_uint64
        lib.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_raw_u64.restype = None
        lib.synth_raw_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                         ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def stream_seed(base: int, config: int = 0, layer: int = 0, tensor: int = 0) -> int:
    """Seed of one tensor's stream, derived from the run's base seed."""
    return int(_load().synth_u64((base ^ (config << 40) ^ (layer << 16) ^ tensor) & (2**64 - 1), 0))


def raw_u64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 stream ``seed``."""
    out = np.empty(count, dtype=np.uint64)
    _load().synth_raw_u64(seed, start, count, out.ctypes.data)
    return out


def normal_f32(seed: int, count: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    """``count`` fp32 draws from N(0, sigma^2): draws ``start ..`` of the stream."""
    out = np.empty(count, dtype=np.float32)
    if count:
        _load().synth_normal_f32(seed, start, count, float(sigma), out.ctypes.data, _threads())
    return out


def choose_channels(seed: int, k: int, n: int) -> np.ndarray:
    """``n`` distinct channels of ``range(k)`` by a seeded partial Fisher-Yates shuffle."""
    perm = list(range(k))
    r = raw_u64(seed, 0, n)
    for i in range(n):
        j = i + int(r[i]) % (k - i)
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(np.array(perm[:n], dtype=np.int64))


def weights(seed: int, n: int, k: int, sigma: float = 0.02) -> np.ndarray:
    """fp32 master weights ``[n][k]`` ~ N(0, sigma^2), row-major."""
    return normal_f32(seed, n * k, sigma).reshape(n, k)


def activations(seed: int, m: int, k: int, n_outliers: int = 0, sigma: float = 1.0,
                factor: float = 20.0) -> np.ndarray:
    """fp32 activations ``[m][k]`` ~ N(0, sigma^2). ``n_outliers`` channels, the same
    for every token, are multiplied by ``factor`` in fp32 after the draw."""
    x = normal_f32(seed, m * k, sigma).reshape(m, k)
    if n_outliers:
        ch = choose_channels(stream_seed(seed, tensor=T_OUTLIER), k, n_outliers)
        x[:, ch] = x[:, ch] * np.float32(factor)
    return x


def outlier_count(k: int) -> int:
    """Outlier channels for a "1 % of channels" workload: round(0.01 * k), halves up."""
    return (k + 50) // 100
