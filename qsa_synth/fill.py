"""GPU fill of the large synthetic tensors (index keys, KV pools).

Builds ``csrc/synth_fill.hip`` into ``_build/libqsasynth.so`` and fills torch
device tensors with exactly the bytes that ``qsa_synth`` generates on the
host. Input generation only; the product library does not use it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import GEOM, HostInputs

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "synth_fill.hip")
_LIB = os.path.join(_HERE, "_build", "libqsasynth.so")
_lib = None

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(force: bool = True) -> str:
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["hipcc", *HIP_FLAGS, _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError("libqsasynth.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB)
        P, i64, i32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64
        lib.synth_fill_index.argtypes = [P, P, i64, i32, i32, u64, P, i32, P, i32, P]
        lib.synth_fill_index.restype = i32
        lib.synth_fill_kv.argtypes = [P, i64, i64, i64, i32, u64, P]
        lib.synth_fill_kv.restype = i32
        _lib = lib
    return _lib


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def fill_index_layer(hi: HostInputs, layer: int, keys, scales, stream=None):
    """Fill device tensors keys u8 [rows][64] and scales (int16/uint16) [rows]
    with layer `layer` of every sequence, packed at row0[b]."""
    import torch
    lib = _load()
    dev = keys.device
    for b in range(hi.wl.batch):
        L = int(hi.lay.ctx[b])
        r0 = int(hi.lay.row0[b])
        planted = torch.from_numpy(np.ascontiguousarray(hi.lay.planted[(layer, b)], np.int32)).to(dev)
        u = torch.from_numpy(np.ascontiguousarray(hi.u[layer, b], np.float32)).to(dev)
        rc = lib.synth_fill_index(ctypes.c_void_p(keys.data_ptr() + r0 * GEOM.idx_dim),
                                  ctypes.c_void_p(scales.data_ptr() + r0 * 2), L, b, layer, hi.wl.seed,
                                  ctypes.c_void_p(planted.data_ptr()), int(planted.numel()),
                                  ctypes.c_void_p(u.data_ptr()), GEOM.block_tokens, _stream_ptr(stream))
        if rc != 0:
            raise RuntimeError("synth_fill_index failed: %d" % rc)
        # keep the small staging tensors alive until the fill has run
        torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()


def fill_kv_rows(dst, slot0: int, n_slots: int, layer: int, seed: int, stream=None):
    """Fill rows [slot0, slot0 + n_slots) of one layer's pool into the device
    tensor `dst` (which starts at row slot0)."""
    lib = _load()
    rc = lib.synth_fill_kv(ctypes.c_void_p(dst.data_ptr()), slot0, n_slots, GEOM.row_elems, layer, seed,
                           _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError("synth_fill_kv failed: %d" % rc)
