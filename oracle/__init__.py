"""CPU oracle of the QSA sparse-attention decode step (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never loads it and
shares no code with it. The arithmetic lives in ``qsa_oracle.c`` (plain C,
single thread, IEEE double); this module only builds it with gcc and passes
numpy arrays to it through ctypes. ``gather_rows`` is the one step written in
numpy: row gathering is plain indexing.

Every function names the passage it follows in its docstring; the C file's
header lists the pages and the readings taken where they are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libqsa_oracle.so")
# A copy instrumented with AddressSanitizer and UndefinedBehaviorSanitizer,
# built with clang so that it shares the ASan runtime of the sanitized host
# build of libqsa (the CPU tests run both under it, tests/test_sanitized.py).
SAN_LIB_PATH = os.path.join(_HERE, "_build", "libqsa_oracle_san.so")
SAN_CC = "/opt/rocm/llvm/bin/clang"
_lib = None


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile qsa_oracle.c with gcc (no fast-math, no FP contraction); with
    sanitize, the instrumented copy with clang."""
    path = SAN_LIB_PATH if sanitize else _LIB_PATH
    os.makedirs(os.path.dirname(path), exist_ok=True)
    if force or not os.path.exists(path):
        tmp = path + ".tmp%d" % os.getpid()
        if sanitize:
            cmd = [SAN_CC, "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                   "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        else:
            cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                   "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if os.environ.get("QSA_ORACLE_SANITIZED") == "1":
        if not os.path.exists(SAN_LIB_PATH):
            raise RuntimeError("the sanitized oracle is not built (%s)" % SAN_LIB_PATH)
        lib = ctypes.CDLL(SAN_LIB_PATH)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.qo_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.qo_decode_e4m3.restype = f64
    lib.qo_decode_f16.argtypes = [ctypes.c_uint16]
    lib.qo_decode_f16.restype = f64
    lib.qo_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.qo_decode_bf16.restype = f64
    lib.qo_encode_f16.argtypes = [f64]
    lib.qo_encode_f16.restype = ctypes.c_uint16
    lib.qo_encode_e4m3.argtypes = [f64]
    lib.qo_encode_e4m3.restype = ctypes.c_uint8
    lib.qo_quantise_key.argtypes = [i32, P, P, P]
    lib.qo_quantise_key.restype = None
    lib.qo_token_scores.argtypes = [i64, i32, i32, P, P, P, P, P]
    lib.qo_token_scores.restype = None
    lib.qo_block_scores.argtypes = [i64, i32, P, P]
    lib.qo_block_scores.restype = None
    lib.qo_forced_mask.argtypes = [i64, i32, i64, i64, P]
    lib.qo_forced_mask.restype = i64
    lib.qo_select_blocks.argtypes = [i64, P, i64, P, P, P]
    lib.qo_select_blocks.restype = i64
    lib.qo_tokens_of_blocks.argtypes = [i64, i32, P, i64, P]
    lib.qo_tokens_of_blocks.restype = i64
    lib.qo_attention.argtypes = [i64, P, P, P, i32, i32, i32, P, f64, P]
    lib.qo_attention.restype = None
    lib.qo_decode_layer.argtypes = [i64, i32, i32, i32, i64, i64, i64, P, P, P, P, P, P, P,
                                    i32, i32, i32, f64, P, P, P, P, P, P]
    lib.qo_decode_layer.restype = i64
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ formats

def decode_e4m3(code: int) -> float:
    """OCP FP8 E4M3FN code -> value (format definition; NaN for S.1111.111)."""
    return _load().qo_decode_e4m3(int(code))


def decode_f16(bits: int) -> float:
    """IEEE binary16 bits -> value."""
    return _load().qo_decode_f16(int(bits))


def decode_bf16(bits: int) -> float:
    """bfloat16 bits -> value (upper half of a binary32)."""
    return _load().qo_decode_bf16(int(bits))


# ---------------------------------------------------------------- the steps

def token_scores(keys, scales, q_idx, w):
    """Indexer score of every cached token of one sequence-layer.

    Follows the mechanism section of the digest page (a resident index of
    compact 66-byte keys is scanned every step) with the score
    s_t = sum_h w_h * ReLU(sigma_t * q_h . k_t) of the workload definition.
    keys u8 [L][D] e4m3 codes, scales u16 [L] fp16 bits, q_idx u16 [H][D] bf16
    bits, w f32 [H]. Returns f32 [L].
    """
    keys = _c(keys, np.uint8)
    scales = _c(scales, np.uint16)
    q_idx = _c(q_idx, np.uint16)
    w = _c(w, np.float32)
    L, D = keys.shape
    H = q_idx.shape[0]
    assert q_idx.shape == (H, D) and scales.shape == (L,) and w.shape == (H,)
    out = np.empty(L, np.float32)
    _load().qo_token_scores(L, H, D, _ptr(keys), _ptr(scales), _ptr(q_idx), _ptr(w), _ptr(out))
    return out


def block_scores(ts, bt: int = 4):
    """C4 block reduce (the article's intro: 4 adjacent tokens form a block):
    max of the fp32 token scores over each block's valid tokens."""
    ts = _c(ts, np.float32)
    L = ts.shape[0]
    out = np.empty((L + bt - 1) // bt, np.float32)
    _load().qo_block_scores(L, bt, _ptr(ts), _ptr(out))
    return out


def forced_mask(L: int, bt: int = 4, sink_blocks: int = 0, tail_tokens: int = 0):
    """Forced blocks: the first sink_blocks blocks and every block holding one
    of the last tail_tokens tokens (the article's sink and tail ring buffer)."""
    n_blk = (L + bt - 1) // bt
    mask = np.zeros(max(n_blk, 1), np.uint8)
    _load().qo_forced_mask(L, bt, sink_blocks, tail_tokens, _ptr(mask))
    return mask[:n_blk]


@dataclass
class Selection:
    blocks: np.ndarray   # int32, ascending
    kth_score: float     # score of the last non-forced block taken (NaN if none)


def select_blocks(bs, K: int, forced=None) -> Selection:
    """Budgeted block selection (digest lead and mechanism sections: at most
    indexer_budget positions; article intro: per C4 block): all blocks when they
    fit, else the forced blocks plus the best K-|F| others by (score desc,
    index asc), returned ascending. Raises ValueError if |F| > K."""
    bs = _c(bs, np.float32)
    n = bs.shape[0]
    fm = None if forced is None else _c(forced, np.uint8)
    sel = np.empty(max(min(n, K), 1), np.int32)
    kth = np.full(1, np.nan, np.float32)
    n_sel = _load().qo_select_blocks(n, _ptr(bs), K, _ptr(fm), _ptr(sel), _ptr(kth))
    if n_sel < 0:
        raise ValueError("forced blocks exceed the budget")
    return Selection(sel[:n_sel].copy(), float(kth[0]))


def tokens_of_blocks(L: int, sel, bt: int = 4):
    """Ascending token positions covered by the selected blocks."""
    sel = _c(sel, np.int32)
    tok = np.empty(max(len(sel) * bt, 1), np.int64)
    n = _load().qo_tokens_of_blocks(L, bt, _ptr(sel), len(sel), _ptr(tok))
    return tok[:n].copy()


def attention(tokens, pt, pool, q, n_kv_heads: int, sm_scale: float):
    """GQA softmax attention of one decode query over the given tokens (the
    attention the article's fast path computes, restricted to the gathered
    set). pool u16 [n_slots][2*n_kv*Dh] bf16 bits (keys of all KV heads, then
    values); pt int32 (or None for slot = token); q u16 [Hq][Dh] bf16 bits.
    Returns f32 [Hq][Dh]."""
    tokens = _c(tokens, np.int64)
    pool = _c(pool, np.uint16)
    q = _c(q, np.uint16)
    Hq, Dh = q.shape
    assert pool.shape[1] == 2 * n_kv_heads * Dh
    ptc = None if pt is None else _c(pt, np.int32)
    out = np.empty((Hq, Dh), np.float32)
    _load().qo_attention(len(tokens), _ptr(tokens), _ptr(ptc), _ptr(pool), Hq, n_kv_heads, Dh,
                         _ptr(q), float(sm_scale), _ptr(out))
    return out


def gather_rows(pool, pt, tokens):
    """Page-table translate and row gather (the article's logical-token to
    physical-slot split; the digest's transfer of only the selected rows):
    row p of the result is pool[pt[tokens[p]]]. Plain numpy indexing."""
    pool = np.asarray(pool)
    return pool[np.asarray(pt)[np.asarray(tokens, np.int64)]]


@dataclass
class LayerResult:
    token_scores: np.ndarray
    block_scores: np.ndarray
    sel: np.ndarray
    kth_score: float
    tokens: np.ndarray
    out: np.ndarray


def decode_layer(keys, scales, q_idx, w, q, pt, pool, *, n_kv_heads: int, budget_tokens: int,
                 sm_scale: float, bt: int = 4, sink_blocks: int = 0, tail_tokens: int = 0) -> LayerResult:
    """One sequence through one QSA layer, in the method's order: score, C4
    reduce, select, expand to tokens, attend through the page table."""
    keys = _c(keys, np.uint8)
    scales = _c(scales, np.uint16)
    q_idx = _c(q_idx, np.uint16)
    w = _c(w, np.float32)
    q = _c(q, np.uint16)
    pt = _c(pt, np.int32)
    pool = _c(pool, np.uint16)
    L, D = keys.shape
    H = q_idx.shape[0]
    Hq, Dh = q.shape
    n_blk = (L + bt - 1) // bt
    ts = np.empty(max(L, 1), np.float32)
    bs = np.empty(max(n_blk, 1), np.float32)
    sel = np.empty(max(n_blk, 1), np.int32)
    kth = np.full(1, np.nan, np.float32)
    ntok = np.zeros(1, np.int64)
    out = np.empty((Hq, Dh), np.float32)
    n_sel = _load().qo_decode_layer(L, H, D, bt, budget_tokens, sink_blocks, tail_tokens,
                                    _ptr(keys), _ptr(scales), _ptr(q_idx), _ptr(w), _ptr(q),
                                    _ptr(pt), _ptr(pool), Hq, n_kv_heads, Dh, float(sm_scale),
                                    _ptr(ts), _ptr(bs), _ptr(sel), _ptr(kth), _ptr(ntok), _ptr(out))
    if n_sel < 0:
        raise ValueError("forced blocks exceed the budget")
    sel = sel[:n_sel].copy()
    return LayerResult(ts[:L].copy(), bs[:n_blk].copy(), sel, float(kth[0]),
                       tokens_of_blocks(L, sel, bt), out)


# ------------------------------------------------------------ append step

def encode_f16(x: float) -> int:
    """Nearest binary16 (ties to even) of a non-negative value, as bits."""
    return int(_load().qo_encode_f16(float(x)))


def encode_e4m3(y: float) -> int:
    """Nearest e4m3 code (ties to even, |y| >= 448 saturates to 448)."""
    return int(_load().qo_encode_e4m3(float(y)))


def quantise_key(x):
    """One index key, float32 [idx_dim] -> (codes u8 [idx_dim], scale bits u16).

    The append step of the memory-ledger section of "双卡RTX4090跑通Qwen3-Next"
    (index, scales and page layout kept together): sigma = fp16(amax / 448),
    code_i = e4m3(x_i / sigma), divisions in binary32."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    codes = np.zeros(x.size, np.uint8)
    s = np.zeros(1, np.uint16)
    _load().qo_quantise_key(x.size, _ptr(x), _ptr(codes), _ptr(s))
    return codes, int(s[0])


def append_token(ctx, row0, pt, slot, keys_layers, scales_layers, pools, new_keys, new_rows):
    """Reference append over host arrays (modified in place).

    For each sequence b with t = ctx[b]: every layer l gets the quantised
    new_keys[l][b] at index row row0[b] + t and new_rows[l][b] at pool slot
    slot[b]; the page table maps t -> slot[b]; the length becomes t + 1.
    Returns the new lengths."""
    out = np.array(ctx, dtype=np.int64).copy()
    for b in range(len(ctx)):
        t = int(ctx[b])
        for l in range(len(keys_layers)):
            c, s = quantise_key(new_keys[l][b])
            keys_layers[l][row0[b] + t] = c
            scales_layers[l][row0[b] + t] = s
            pools[l][slot[b]] = new_rows[l][b]
        pt[b, t] = slot[b]
        out[b] = t + 1
    return out


# --------------------------------------------------------------- hot cache

def hot_cache_update(hot_map, owner, tokens, b: int, H: int):
    """One sequence-layer's hot-cache update before attention (test reference,
    plain Python).

    The memory-ledger section of "双卡RTX4090跑通Qwen3-Next" keeps only hot
    rows on the GPU and moves missing rows back from pinned host memory on
    demand, with a per-layer mapping from logical tokens to cache slots. Here
    the cache of sequence b holds H rows, global slot ids b*H .. b*H + H - 1:
      hot_map[t]  = slot id holding logical token t, or -1;
      owner[h]    = logical token held by local slot h, or -1.
    `tokens` are this step's selected tokens in ascending order. Tokens already
    cached are hits and keep their slots. The misses, in ascending token
    order, take the slots not used by a hit this step, in ascending slot
    order; a slot's previous token loses its mapping. Returns the list of
    (token, local slot) fetches, in that order. hot_map and owner are updated
    in place."""
    used = [False] * H
    misses = []
    for t in tokens:
        h = int(hot_map[t])
        if h >= 0:
            used[h - b * H] = True
        else:
            misses.append(int(t))
    free = [h for h in range(H) if not used[h]]
    assert len(free) >= len(misses), "hot cache smaller than the selection"
    fetches = []
    for t, h in zip(misses, free):
        old = int(owner[h])
        if old >= 0:
            hot_map[old] = -1
        owner[h] = t
        hot_map[t] = b * H + h
        fetches.append((t, h))
    return fetches


# ------------------------------------------------------------ slot leases

class SlotPoolModel:
    """Reference model of slot leases (test infrastructure, plain Python).

    The memory-ledger section of "双卡RTX4090跑通Qwen3-Next" lets requests
    finish, be cancelled and hand their cache to new requests safely through
    leases, generation markers and a tail ring buffer, after which the cache
    capacity and slots return to their initial values. The model:
      - the pool has n_slots physical slots, each with a generation counter
        starting at 0; free slots are handed out lowest first;
      - a lease (one request) may keep a tail ring of R slots, taken when the
        lease opens: token t is written to ring slot ring[t % R]; when token
        t >= R arrives, token t - R leaves the ring and moves to a body slot
        taken from the pool (its row is copied ring -> body first);
      - without a ring (R = 0) every token takes a body slot directly;
      - closing a lease returns every slot it holds and increments each one's
        generation, so that a page-table entry recorded under the old
        generation is recognisably stale.
    next_token returns the plan of one appended token:
      (slot, generation, spill) with spill = None or (token, from_slot,
      to_slot, to_generation)."""

    def __init__(self, n_slots: int):
        self.n = n_slots
        self.gen = [0] * n_slots
        self.free = list(range(n_slots))          # kept sorted
        self.leases = {}
        self.next_id = 1

    def _take(self):
        if not self.free:
            raise MemoryError("pool exhausted")
        return self.free.pop(0)

    def _give(self, s):
        self.gen[s] += 1
        self.free.append(s)
        self.free.sort()

    def open(self, ring: int) -> int:
        if ring > len(self.free):
            raise MemoryError("pool exhausted")
        lid = self.next_id
        self.next_id += 1
        self.leases[lid] = {"ring": [self._take() for _ in range(ring)], "body": [], "t": 0}
        return lid

    def next_token(self, lid: int):
        L = self.leases[lid]
        t, R = L["t"], len(L["ring"])
        if R == 0:
            s = self._take()
            L["body"].append(s)
            L["t"] += 1
            return s, self.gen[s], None
        spill = None
        s = L["ring"][t % R]
        if t >= R:
            to = self._take()
            L["body"].append(to)
            spill = (t - R, s, to, self.gen[to])
        L["t"] += 1
        return s, self.gen[s], spill

    def close(self, lid: int):
        L = self.leases.pop(lid)
        for s in L["ring"] + L["body"]:
            self._give(s)

    def free_slots(self) -> int:
        return len(self.free)


# ----------------------------------------------------- multi-query scoring

def multi_block_scores(keys, scales, q_idx, w, pos, n_blk_out, bt: int = 4):
    """Block scores of several queries of one sequence against its index (for
    prefill or chunked decode), each query seeing the tokens up to and
    including its own position pos[i] (causal). Query i's block j is the max
    of its token scores over the tokens of j that it sees, -inf when it sees
    none of them. The scores themselves are the single-query scores of the
    indexer (digest, mechanism section; the workload's formula), so each row
    is `block_scores(token_scores(keys[:pos+1], ...))` padded with -inf.
    Returns float32 [Q][n_blk_out]."""
    Q = len(pos)
    out = np.full((Q, n_blk_out), -np.inf, np.float32)
    for i in range(Q):
        n = int(pos[i]) + 1
        ts = token_scores(keys[:n], scales[:n], q_idx[i], w[i])
        bs = block_scores(ts, bt)
        out[i, :len(bs)] = bs
    return out
