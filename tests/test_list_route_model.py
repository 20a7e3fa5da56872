"""The long-context selection's exactness argument, on the CPU.

The GPU route keeps, per scoring chunk, a list of the chunk's eligible blocks
whose 12-bit key bin is at least a threshold bin (at least m of them, at most
cap, or only the bins above a crowded one), selects the r-th largest T_U of
the union, and re-reads only the chunks whose list is incomplete, wholly at
or above T_U, and whose threshold lies above T_U. This model runs those
steps in numpy (composites key << 32 | ~index, the order key of the kernels)
and checks that the result is the oracle's selection for random, tied,
constant, mostly-zero, clustered and one-bin scores; it also checks that the
re-read path is taken in some cases, so the test reaches it.
"""
import numpy as np
import pytest

import oracle

HB = 12
SH = 32 - HB
M64 = np.uint64(0xFFFFFFFF)


def order_keys(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = np.where((u & np.uint64(0x7FFFFFFF)) == 0, np.uint64(0), u)
    neg = (u & np.uint64(0x80000000)) != 0
    return np.where(neg, (~u) & M64, u | np.uint64(0x80000000)).astype(np.uint64)


def chunk_list(keys, idx, m, cap):
    """(threshold bin, complete, composites) of one chunk's eligible blocks."""
    bins = (keys >> np.uint64(SH)).astype(np.int64)
    comps = (keys << np.uint64(32)) | (M64 - idx.astype(np.uint64))
    tot = len(keys)
    if tot < m:
        return 0, True, comps
    h = np.bincount(bins, minlength=1 << HB)
    from_top = np.cumsum(h[::-1])
    bx = (1 << HB) - 1 - int(np.argmax(from_top >= m))
    cum = int(from_top[(1 << HB) - 1 - bx])
    if cum <= cap:
        theta, complete = bx, cum == tot
    else:
        theta, complete = bx + 1, False
    return theta, complete, comps[bins >= theta]


def list_route(scores, K, sink, tail_first, chunk_blocks, m, cap):
    n = len(scores)
    j = np.arange(n)
    el = (j >= sink) & (j < tail_first)
    forced = j[~el]
    r = K - len(forced)
    keys = order_keys(scores)
    lists = []
    for c0 in range(0, n, chunk_blocks):
        sl = slice(c0, min(c0 + chunk_blocks, n))
        e = el[sl]
        lists.append(chunk_list(keys[sl][e], j[sl][e], m, cap))
    if r <= 0:
        return forced, 0
    pool = np.concatenate([l[2] for l in lists])
    bounded = len(pool) >= r
    tu = np.sort(pool)[::-1][r - 1] if bounded else np.uint64(0)
    needy = []
    for c, (theta, complete, comps) in enumerate(lists):
        if complete:
            continue
        if bounded and not ((np.uint64(theta) << np.uint64(SH)) > (tu >> np.uint64(32))
                            and np.all(comps >= tu)):
            continue
        needy.append(c)
    for c in needy:
        theta = lists[c][0]
        sl = slice(c * chunk_blocks, min((c + 1) * chunk_blocks, n))
        e = el[sl]
        k, ix = keys[sl][e], j[sl][e]
        comps = (k << np.uint64(32)) | (M64 - ix.astype(np.uint64))
        add = ((k >> np.uint64(SH)) < np.uint64(theta)) & ((comps >= tu) if bounded else True)
        pool = np.concatenate([pool, comps[add]])
    t = np.sort(pool)[::-1][r - 1]
    chosen = (M64 - (pool[pool >= t] & M64)).astype(np.int64)
    return np.union1d(chosen, forced), len(needy)


def cases():
    rng = np.random.default_rng(12)
    for trial in range(240):
        n = int(rng.integers(16, 2500))
        K = int(rng.integers(4, 160))
        cb = int(rng.choice([8, 32, 128, 512]))
        sink = int(rng.integers(0, 3))
        tail = int(rng.integers(0, 12))
        L = 4 * n - int(rng.integers(0, 4))
        tail_first = n if tail == 0 else max(0, L - tail) // 4
        n_forced = min(sink, n) + max(0, n - max(tail_first, min(sink, n)))
        if n <= K or n_forced > K:
            continue
        kind = trial % 6
        if kind == 0:
            s = rng.standard_normal(n)
        elif kind == 1:
            s = np.round(rng.standard_normal(n) * 2)
        elif kind == 2:
            s = np.full(n, 1.5)
        elif kind == 3:
            s = np.where(rng.random(n) < 0.1, rng.random(n), 0.0)
        elif kind == 4:
            s = rng.standard_normal(n)
            a = int(rng.integers(0, n))
            s[a:a + 300] += 5.0
        else:
            s = rng.standard_normal(n) * 1e-3 + 1.0
        n_chunks = (n + cb - 1) // cb
        m = max(4, min(64, (3 * K + n_chunks - 1) // n_chunks))
        cap = 2 * m if trial % 3 else int(rng.choice([m, m + 2, 128]))
        yield np.asarray(s, np.float32), L, K, sink, tail, tail_first, cb, m, cap


def test_list_route_selects_what_the_oracle_selects():
    re_read = 0
    checked = 0
    for s, L, K, sink, tail, tail_first, cb, m, cap in cases():
        got, n_needy = list_route(s, K, sink, tail_first, cb, m, cap)
        ref = oracle.select_blocks(s, K, oracle.forced_mask(L, 4, sink, tail)).blocks
        assert np.array_equal(got, np.asarray(ref)), (L, K, cb, m, cap)
        re_read += n_needy > 0
        checked += 1
    assert checked > 150
    assert re_read > 10          # the re-read path was exercised


def test_full_lists_bound_the_chunks_re_read():
    """Lists of at least m entries (no crowded bin): at most r / m chunks are
    re-read."""
    rng = np.random.default_rng(3)
    for _ in range(40):
        n, K, cb = 4096, 128, 64
        s = rng.standard_normal(n).astype(np.float32)
        a = int(rng.integers(0, n - 600))
        s[a:a + 600] += 6.0
        m = max(4, (3 * K + n // cb - 1) // (n // cb))
        got, n_needy = list_route(s, K, 0, n, cb, m, 128)
        assert n_needy <= K // m
        ref = oracle.select_blocks(s, K, oracle.forced_mask(4 * n, 4, 0, 0)).blocks
        assert np.array_equal(got, np.asarray(ref))
