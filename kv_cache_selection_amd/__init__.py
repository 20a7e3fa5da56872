"""Python binding of libqsa (the QSA sparse-attention decode step on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libqsa.so``. Functions keep the C names (``qsa_index_score`` ...), take
torch tensors (device memory, or pinned host memory for the KV pool of the
offload path) or raw integer addresses, and raise ``QsaError`` on a status
other than QSA_OK. Importing fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os

try:  # load torch's HIP runtime first so that one runtime serves both
    import torch  # noqa: F401
except ImportError:  # pragma: no cover
    torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
# QSA_LIBRARY names another build of the same library (the tests' sanitized
# host build); by default the in-tree libqsa.so is loaded.
LIB_PATH = os.environ.get("QSA_LIBRARY") or os.path.join(_HERE, "libqsa.so")

QSA_OK, QSA_ERR_INVALID_ARGUMENT, QSA_ERR_UNSUPPORTED, QSA_ERR_WORKSPACE_TOO_SMALL, QSA_ERR_HIP, QSA_ERR_OUT_OF_SLOTS = range(6)
QSA_KV_DEVICE, QSA_KV_HOST_PINNED = 0, 1
QSA_FLAG_BAD_SLOT, QSA_FLAG_BAD_INDEX_ROWS, QSA_FLAG_BAD_CTX_LEN, QSA_FLAG_BAD_N_TOK = 1, 2, 4, 8
QSA_MAX_SIDE_STREAMS = 8

# Every symbol include/libqsa.h declares.
EXPORTS = ("qsa_index_score", "qsa_topk_blocks", "qsa_gather_kv", "qsa_sparse_decode", "qsa_decode_step",
           "qsa_step_events_create", "qsa_step_events_destroy", "qsa_read_flags", "qsa_decode_step_static",
           "qsa_append_token", "qsa_hot_reset", "qsa_move_tokens", "qsa_check_generations", "qsa_index_score_multi",
           "qsa_pool_create", "qsa_pool_destroy", "qsa_pool_open", "qsa_pool_next", "qsa_pool_close",
           "qsa_pool_free_slots", "qsa_pool_generations",
           "qsa_workspace_size", "qsa_layer_bytes", "qsa_status_string")


class QsaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32), ("block_tokens", ctypes.c_int32),
                ("budget_tokens", ctypes.c_int32), ("sink_blocks", ctypes.c_int32),
                ("tail_tokens", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


class Batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("ctx_len", ctypes.c_void_p),
                ("idx_row0", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("pt_stride", ctypes.c_int64),
                ("n_slots", ctypes.c_int64), ("n_idx_rows", ctypes.c_int64)]


class AppendLayer(ctypes.Structure):
    _fields_ = [("new_idx_key", ctypes.c_void_p), ("new_kv_row", ctypes.c_void_p), ("idx_keys", ctypes.c_void_p),
                ("idx_scales", ctypes.c_void_p), ("kv_pool", ctypes.c_void_p)]


class SlotPlan(ctypes.Structure):
    _fields_ = [("token", ctypes.c_int64), ("slot", ctypes.c_int32), ("generation", ctypes.c_uint32),
                ("spill_token", ctypes.c_int64), ("spill_from", ctypes.c_int32), ("spill_to", ctypes.c_int32),
                ("spill_generation", ctypes.c_uint32)]


class Layer(ctypes.Structure):
    _fields_ = [("idx_keys", ctypes.c_void_p), ("idx_scales", ctypes.c_void_p), ("q_idx", ctypes.c_void_p),
                ("w_idx", ctypes.c_void_p), ("q", ctypes.c_void_p), ("kv_pool", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("out", ctypes.c_void_p), ("sel_blocks", ctypes.c_void_p),
                ("n_sel", ctypes.c_void_p), ("hot", ctypes.c_void_p), ("score_events", ctypes.c_void_p * 2)]


class HotCache(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_void_p), ("map", ctypes.c_void_p), ("owner", ctypes.c_void_p),
                ("hot_slots", ctypes.c_int32), ("n_miss", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libqsa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    CP, BP = ctypes.POINTER(Config), ctypes.POINTER(Batch)
    lib.qsa_index_score.argtypes = [CP, BP, P, P, P, P, P, P, i64, P]
    lib.qsa_topk_blocks.argtypes = [CP, BP, P, i64, P, P, P, P, sz, P]
    lib.qsa_gather_kv.argtypes = [CP, BP, P, P, P, i32, P, P, P]
    lib.qsa_sparse_decode.argtypes = [CP, i32, P, P, P, P, P, sz, P]
    lib.qsa_append_token.argtypes = [CP, BP, ctypes.POINTER(AppendLayer), i32, i32, P, P, P, P, P, P]
    lib.qsa_index_score_multi.argtypes = [CP, BP, i32, P, P, P, P, P, P, i64, P]
    lib.qsa_move_tokens.argtypes = [BP, ctypes.POINTER(ctypes.c_void_p), i32, i32, P, P, P, P, P, P]
    lib.qsa_check_generations.argtypes = [BP, P, P, P, P, P]
    lib.qsa_pool_create.argtypes = [i64, ctypes.POINTER(ctypes.c_void_p)]
    lib.qsa_pool_destroy.argtypes = [P]
    lib.qsa_pool_destroy.restype = None
    lib.qsa_pool_open.argtypes = [P, i32, ctypes.POINTER(ctypes.c_int32)]
    lib.qsa_pool_next.argtypes = [P, i32, ctypes.POINTER(SlotPlan)]
    lib.qsa_pool_close.argtypes = [P, i32]
    lib.qsa_pool_free_slots.argtypes = [P]
    lib.qsa_pool_free_slots.restype = i64
    lib.qsa_pool_generations.argtypes = [P, P]
    lib.qsa_hot_reset.argtypes = [BP, ctypes.POINTER(HotCache), P]
    lib.qsa_decode_step.argtypes = [CP, BP, ctypes.POINTER(Layer), i32, i32, P, sz, P,
                                    ctypes.POINTER(ctypes.c_void_p), i32, P]
    lib.qsa_step_events_create.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_void_p)]
    lib.qsa_step_events_destroy.argtypes = [P]
    lib.qsa_step_events_destroy.restype = None
    lib.qsa_read_flags.argtypes = [P, P, P]
    lib.qsa_decode_step_static.argtypes = [CP, BP, ctypes.POINTER(Layer), i32, i32, P,
                                           ctypes.POINTER(ctypes.c_void_p), i32, P]
    for f in ("qsa_index_score", "qsa_topk_blocks", "qsa_gather_kv", "qsa_sparse_decode", "qsa_decode_step",
              "qsa_step_events_create", "qsa_read_flags", "qsa_decode_step_static",
              "qsa_append_token", "qsa_hot_reset", "qsa_move_tokens", "qsa_check_generations", "qsa_index_score_multi", "qsa_pool_create",
              "qsa_pool_open", "qsa_pool_next", "qsa_pool_close", "qsa_pool_generations"):
        getattr(lib, f).restype = i32
    lib.qsa_workspace_size.argtypes = [CP, i32, i32, i32, i32]
    lib.qsa_workspace_size.restype = sz
    lib.qsa_layer_bytes.argtypes = [CP, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.qsa_layer_bytes.restype = None
    lib.qsa_status_string.argtypes = [i32]
    lib.qsa_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def _p(x):
    """Address of a tensor (data_ptr), an int, or None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn, st):
    if st != QSA_OK:
        raise QsaError(fn, st)


def status_string(st: int) -> str:
    return lib.qsa_status_string(st).decode()


def make_config(budget_tokens, sink_blocks=0, tail_tokens=0, sm_scale=1.0 / 16.0, n_q_heads=16, n_kv_heads=2,
                head_dim=256, idx_heads=4, idx_dim=64, block_tokens=4) -> Config:
    return Config(n_q_heads, n_kv_heads, head_dim, idx_heads, idx_dim, block_tokens, budget_tokens, sink_blocks,
                  tail_tokens, sm_scale)


def make_batch(batch, max_ctx, ctx_len, idx_row0=None, page_table=None, pt_stride=0, n_slots=0,
               n_idx_rows=None) -> Batch:
    """The structs hold raw addresses only, so every tensor passed here is
    also kept referenced by the returned struct: it cannot be freed (and its
    memory reused) while the struct is alive."""
    if idx_row0 is not None and n_idx_rows is None:
        raise ValueError("n_idx_rows is required with idx_row0")
    b = Batch(batch, max_ctx, _p(ctx_len), _p(idx_row0), _p(page_table), pt_stride, n_slots, n_idx_rows or 0)
    b._keep = (ctx_len, idx_row0, page_table)
    return b


def qsa_workspace_size(cfg: Config, batch: int, max_ctx: int, n_layers: int = 1,
                       kv_location: int = QSA_KV_DEVICE) -> int:
    return lib.qsa_workspace_size(ctypes.byref(cfg), batch, max_ctx, n_layers, kv_location)


def qsa_layer_bytes(cfg: Config, ctx: int, n_tok: int):
    a, b = ctypes.c_int64(), ctypes.c_int64()
    lib.qsa_layer_bytes(ctypes.byref(cfg), ctx, n_tok, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def qsa_index_score(cfg, batch, idx_keys, idx_scales, q_idx, w_idx, token_scores, block_scores, bs_stride,
                    stream=None):
    _check("qsa_index_score", lib.qsa_index_score(ctypes.byref(cfg), ctypes.byref(batch), _p(idx_keys),
                                                  _p(idx_scales), _p(q_idx), _p(w_idx), _p(token_scores),
                                                  _p(block_scores), bs_stride, _stream(stream)))


def qsa_topk_blocks(cfg, batch, block_scores, bs_stride, sel_blocks, n_sel, n_tok, workspace, workspace_bytes,
                    stream=None):
    _check("qsa_topk_blocks", lib.qsa_topk_blocks(ctypes.byref(cfg), ctypes.byref(batch), _p(block_scores),
                                                  bs_stride, _p(sel_blocks), _p(n_sel), _p(n_tok), _p(workspace),
                                                  workspace_bytes, _stream(stream)))


def qsa_gather_kv(cfg, batch, sel_blocks, n_sel, kv_pool, kv_location, kv_out, n_tok, stream=None):
    _check("qsa_gather_kv", lib.qsa_gather_kv(ctypes.byref(cfg), ctypes.byref(batch), _p(sel_blocks), _p(n_sel),
                                              _p(kv_pool), kv_location, _p(kv_out), _p(n_tok), _stream(stream)))


def qsa_sparse_decode(cfg, batch_size, q, kv, n_tok, out, workspace, workspace_bytes, stream=None):
    _check("qsa_sparse_decode", lib.qsa_sparse_decode(ctypes.byref(cfg), batch_size, _p(q), _p(kv), _p(n_tok),
                                                      _p(out), _p(workspace), workspace_bytes, _stream(stream)))


def make_layer(idx_keys, idx_scales, q_idx, w_idx, q, kv_pool, out, page_table=None, sel_blocks=None,
               n_sel=None, score_events=None, hot=None) -> Layer:
    ev = (ctypes.c_void_p * 2)(*(score_events or (None, None)))
    hot_ptr = ctypes.cast(ctypes.pointer(hot), ctypes.c_void_p).value if hot is not None else None
    lay = Layer(_p(idx_keys), _p(idx_scales), _p(q_idx), _p(w_idx), _p(q), _p(kv_pool), _p(page_table), _p(out),
                _p(sel_blocks), _p(n_sel), hot_ptr, ev)
    lay._keep = (idx_keys, idx_scales, q_idx, w_idx, q, kv_pool, page_table, out, sel_blocks, n_sel, hot)
    return lay


def make_hot_cache(rows, map_, owner, hot_slots, n_miss=None) -> HotCache:
    """A layer's hot row cache: rows [B][hot_slots][row_bytes], map [B][pt_stride]
    and owner [B][hot_slots] int32, optional n_miss [B] int32 (device)."""
    hc = HotCache(_p(rows), _p(map_), _p(owner), int(hot_slots), _p(n_miss))
    hc._keep = (rows, map_, owner, n_miss)
    return hc


def qsa_hot_reset(batch, hot, stream=None):
    _check("qsa_hot_reset", lib.qsa_hot_reset(ctypes.byref(batch), ctypes.byref(hot), _stream(stream)))


class StepEvents:
    """The caller-owned event set of the overlapped schedules
    (qsa_step_events_create / _destroy), made on the current device."""

    def __init__(self, max_layers: int, max_side: int):
        h = ctypes.c_void_p()
        _check("qsa_step_events_create", lib.qsa_step_events_create(int(max_layers), int(max_side), ctypes.byref(h)))
        self._h = h
        self.max_layers, self.max_side = int(max_layers), int(max_side)

    @property
    def handle(self):
        return self._h.value

    def destroy(self):
        if self._h:
            lib.qsa_step_events_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _side_array(side):
    if side is None:
        side = ()
    elif not isinstance(side, (list, tuple)):
        side = (side,)
    sarr = (ctypes.c_void_p * max(len(side), 1))(*[_stream(x) for x in side])
    return (sarr if side else None), len(side)


def qsa_decode_step(cfg, batch, layers, kv_location, workspace, workspace_bytes, compute=None, side=None,
                    events=None):
    """`side`: None, one stream, or a sequence of streams (the side streams of
    the overlapped schedules); None or an empty sequence serialises the step
    on `compute`. `events`: a StepEvents (needed by the schedules that order
    several streams), or None."""
    # the array copies the structs; `layers` keeps the tensors they point to alive
    arr = (Layer * len(layers))(*layers)
    sarr, n_side = _side_array(side)
    _check("qsa_decode_step", lib.qsa_decode_step(ctypes.byref(cfg), ctypes.byref(batch), arr, len(layers),
                                                  kv_location, _p(workspace), workspace_bytes, _stream(compute),
                                                  sarr, n_side, events.handle if events is not None else None))


QSA_STATIC_SCRATCH_BYTES = 64 << 20


def qsa_decode_step_static(cfg, batch, layers, kv_location, compute=None, side=None, events=None):
    """qsa_decode_step with the library's static scratch as the workspace
    (allocates nothing; up to QSA_STATIC_SCRATCH_BYTES of workspace need)."""
    arr = (Layer * len(layers))(*layers)
    sarr, n_side = _side_array(side)
    _check("qsa_decode_step_static", lib.qsa_decode_step_static(
        ctypes.byref(cfg), ctypes.byref(batch), arr, len(layers), kv_location, _stream(compute), sarr, n_side,
        events.handle if events is not None else None))


def qsa_read_flags(workspace, flags_out, stream=None):
    """Enqueue a copy of the workspace's flags word (QSA_FLAG_*) into the
    one-element int32/uint32 device tensor flags_out."""
    _check("qsa_read_flags", lib.qsa_read_flags(_p(workspace), _p(flags_out), _stream(stream)))


def make_append_layer(new_idx_key, new_kv_row, idx_keys, idx_scales, kv_pool) -> AppendLayer:
    lay = AppendLayer(_p(new_idx_key), _p(new_kv_row), _p(idx_keys), _p(idx_scales), _p(kv_pool))
    lay._keep = (new_idx_key, new_kv_row, idx_keys, idx_scales, kv_pool)
    return lay


def qsa_append_token(cfg, batch, layers, kv_location, new_slot, page_table, ctx_len_out=None, stream=None,
                     new_gen=None, tok_gen=None):
    arr = (AppendLayer * len(layers))(*layers)
    _check("qsa_append_token", lib.qsa_append_token(ctypes.byref(cfg), ctypes.byref(batch), arr, len(layers),
                                                    kv_location, _p(new_slot), _p(page_table), _p(ctx_len_out),
                                                    _p(new_gen), _p(tok_gen), _stream(stream)))


def qsa_move_tokens(batch, kv_pools, kv_location, token, to_slot, page_table, to_gen=None, tok_gen=None,
                    stream=None):
    arr = (ctypes.c_void_p * len(kv_pools))(*[_p(x) for x in kv_pools])
    _check("qsa_move_tokens", lib.qsa_move_tokens(ctypes.byref(batch), arr, len(kv_pools), kv_location, _p(token),
                                                  _p(to_slot), _p(to_gen), _p(page_table), _p(tok_gen),
                                                  _stream(stream)))


def qsa_check_generations(batch, page_table, tok_gen, slot_gen, stale, stream=None):
    _check("qsa_check_generations", lib.qsa_check_generations(ctypes.byref(batch), _p(page_table), _p(tok_gen),
                                                              _p(slot_gen), _p(stale), _stream(stream)))


class SlotPool:
    """The library's host-side slot pool (qsa_pool_*)."""

    def __init__(self, n_slots: int):
        h = ctypes.c_void_p()
        _check("qsa_pool_create", lib.qsa_pool_create(int(n_slots), ctypes.byref(h)))
        self._h = h
        self.n_slots = int(n_slots)

    def close_pool(self):
        if self._h:
            lib.qsa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close_pool()
        except Exception:
            pass

    def open(self, ring: int) -> int:
        lid = ctypes.c_int32()
        _check("qsa_pool_open", lib.qsa_pool_open(self._h, int(ring), ctypes.byref(lid)))
        return lid.value

    def next_token(self, lease: int) -> SlotPlan:
        plan = SlotPlan()
        _check("qsa_pool_next", lib.qsa_pool_next(self._h, int(lease), ctypes.byref(plan)))
        return plan

    def close(self, lease: int):
        _check("qsa_pool_close", lib.qsa_pool_close(self._h, int(lease)))

    def free_slots(self) -> int:
        return int(lib.qsa_pool_free_slots(self._h))

    def generations(self):
        import numpy as np
        g = np.zeros(self.n_slots, np.uint32)
        _check("qsa_pool_generations", lib.qsa_pool_generations(self._h, ctypes.c_void_p(g.ctypes.data)))
        return g


def qsa_index_score_multi(cfg, batch, n_queries, idx_keys, idx_scales, q_idx, w_idx, q_pos, block_scores, bs_stride,
                          stream=None):
    _check("qsa_index_score_multi", lib.qsa_index_score_multi(ctypes.byref(cfg), ctypes.byref(batch), int(n_queries),
                                                              _p(idx_keys), _p(idx_scales), _p(q_idx), _p(w_idx),
                                                              _p(q_pos), _p(block_scores), int(bs_stride),
                                                              _stream(stream)))
