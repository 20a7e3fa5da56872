"""Host C version of the generator's two large streams (index keys, KV rows).

``csrc/synth_host.c`` produces the same bytes as ``index_keys`` and
``kv_rows`` in this package's numpy code (checked by the test suite), about
two orders of magnitude faster, so that large samples can be regenerated on
the CPU. Input generation only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import GEOM, Geometry

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "synth_host.c")
_LIB = os.path.join(_HERE, "_build", "libqsasynth_host.so")
_lib = None


def build(force: bool = True) -> str:
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P, i64, i32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64
        lib.synth_index_keys.argtypes = [u64, i32, i32, i64, i64, P, i32, P, i32, P, P]
        lib.synth_index_keys.restype = None
        lib.synth_kv_rows.argtypes = [u64, i32, P, i64, i64, P]
        lib.synth_kv_rows.restype = None
        lib.synth_f32_to_f16.argtypes = [ctypes.c_float]
        lib.synth_f32_to_f16.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def index_keys(seed: int, layer: int, b: int, t0: int, t1: int, planted, u, g: Geometry = GEOM):
    """Same result as ``qsa_synth.index_keys``: (codes u8 [n][64], scale bits u16 [n])."""
    assert g.idx_dim == 64
    lib = _load()
    n = t1 - t0
    codes = np.empty((n, g.idx_dim), np.uint8)
    sig = np.empty(n, np.uint16)
    pl = np.ascontiguousarray(planted, dtype=np.int32)
    uu = np.ascontiguousarray(u, dtype=np.float32)
    assert uu.shape == (g.idx_dim,)
    if n > 0:
        lib.synth_index_keys(seed, layer, b, t0, t1, _ptr(pl), len(pl), _ptr(uu), g.block_tokens, _ptr(codes),
                             _ptr(sig))
    return codes, sig


def kv_rows(seed: int, layer: int, slots, g: Geometry = GEOM):
    """Same result as ``qsa_synth.kv_rows``: bf16 bits [len(slots)][row_elems]."""
    lib = _load()
    s = np.ascontiguousarray(slots, dtype=np.int64).reshape(-1)
    out = np.empty((len(s), g.row_elems), np.uint16)
    if len(s):
        lib.synth_kv_rows(seed, layer, _ptr(s), len(s), g.row_elems, _ptr(out))
    return out


def f32_to_f16_bits(x: float) -> int:
    return int(_load().synth_f32_to_f16(x))
