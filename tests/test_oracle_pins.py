"""Pins of the CPU oracle against facts that do not come from the oracle itself:
library decoders and routines, closed forms, invariants and brute force on
tiny inputs. Each test names the passage or the mathematics it rests on.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ formats

def test_e4m3_decode_exhaustive_matches_torch():
    """All 256 OCP E4M3FN codes against torch.float8_e4m3fn (a library decoder)."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.decode_e4m3(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3_named_values():
    """Named points of the format: max 448, smallest normal 2^-6, smallest subnormal 2^-9."""
    assert oracle.decode_e4m3(0x7E) == 448.0
    assert oracle.decode_e4m3(0xFE) == -448.0
    assert oracle.decode_e4m3(0x08) == 2.0 ** -6
    assert oracle.decode_e4m3(0x01) == 2.0 ** -9
    assert oracle.decode_e4m3(0x07) == 7 * 2.0 ** -9
    assert oracle.decode_e4m3(0x38) == 1.0
    assert oracle.decode_e4m3(0x00) == 0.0


def test_f16_decode_exhaustive_matches_numpy():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([oracle.decode_f16(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_bf16_decode_exhaustive_matches_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


# ------------------------------------------------------------ test helpers

def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e4m3_values(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bf16_values(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _random_index(rng, L, H=4, D=64):
    codes = rng.integers(0, 256, size=(L, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN codes
    scales = np.float16(rng.uniform(0.001, 0.02, size=L)).view(np.uint16)
    q_idx = _bf16_bits(rng.standard_normal((H, D)))
    return codes, scales, q_idx


# --------------------------------------------------------- token scores

def test_token_score_one_hot_weight_is_relu_of_library_dot():
    """w = e_h reduces the score to ReLU(sigma * q_h . k): a single dot product,
    computed here with numpy on library-decoded operands."""
    rng = np.random.default_rng(1)
    codes, scales, q_idx = _random_index(rng, 300)
    kv = _e4m3_values(codes)
    qv = _bf16_values(q_idx)
    sig = scales.view(np.float16).astype(np.float64)
    for h in range(4):
        w = np.zeros(4, np.float32)
        w[h] = 1.0
        got = oracle.token_scores(codes, scales, q_idx, w)
        ref = np.maximum(0.0, sig * (kv @ qv[h]))
        np.testing.assert_allclose(got, ref.astype(np.float32), rtol=1e-7, atol=0)
        assert (got > 0).any() and (got == 0).any()


def test_token_score_linear_in_weights():
    """s(w1 + w2) = s(w1) + s(w2): the heads combine by a weighted sum."""
    rng = np.random.default_rng(2)
    codes, scales, q_idx = _random_index(rng, 257)
    w1 = rng.uniform(0, 1, 4).astype(np.float32)
    w2 = rng.uniform(0, 1, 4).astype(np.float32)
    s1 = oracle.token_scores(codes, scales, q_idx, w1).astype(np.float64)
    s2 = oracle.token_scores(codes, scales, q_idx, w2).astype(np.float64)
    s12 = oracle.token_scores(codes, scales, q_idx, (w1.astype(np.float64) + w2).astype(np.float32))
    np.testing.assert_allclose(s12, s1 + s2, rtol=3e-7, atol=1e-30)


def test_token_score_relu_sign_and_scale():
    """For one head, s(q) + s(-q) = |sigma q.k| (the ReLU keeps one sign), and the
    score is linear in the per-token scale (power-of-two scaling is exact)."""
    rng = np.random.default_rng(3)
    codes, scales, q_idx = _random_index(rng, 200)
    w = np.array([1, 0, 0, 0], np.float32)
    neg = q_idx ^ np.uint16(0x8000)
    sp = oracle.token_scores(codes, scales, q_idx, w).astype(np.float64)
    sn = oracle.token_scores(codes, scales, neg, w).astype(np.float64)
    d = _e4m3_values(codes) @ _bf16_values(q_idx)[0] * scales.view(np.float16).astype(np.float64)
    np.testing.assert_allclose(sp + sn, np.abs(d), rtol=1e-7)
    assert np.all((sp == 0) | (sn == 0))
    s2 = (scales.view(np.float16) * np.float16(2)).view(np.uint16)
    w4 = rng.uniform(0, 1, 4).astype(np.float32)
    np.testing.assert_array_equal(oracle.token_scores(codes, s2, q_idx, w4),
                                  2 * oracle.token_scores(codes, scales, q_idx, w4))


def test_token_score_zero_query_and_zero_scale():
    rng = np.random.default_rng(4)
    codes, scales, q_idx = _random_index(rng, 64)
    w = rng.uniform(0, 1, 4).astype(np.float32)
    assert not oracle.token_scores(codes, scales, np.zeros_like(q_idx), w).any()
    assert not oracle.token_scores(codes, np.zeros_like(scales), q_idx, w).any()


def test_token_score_integer_exact():
    """Integer-valued keys and queries with a power-of-two scale: every partial
    sum is an exact integer multiple of the scale, so the score is known exactly
    (Python integers, brute force)."""
    rng = np.random.default_rng(5)
    int_codes = {1.0: 0x38, 2.0: 0x40, 3.0: 0x44, 4.0: 0x48, 0.0: 0x00}
    vals = rng.choice([-4, -3, -2, -1, 0, 1, 2, 3, 4], size=(50, 64))
    codes = np.array([[int_codes[abs(float(v))] | (0x80 if v < 0 else 0) for v in row] for row in vals], np.uint8)
    qi = rng.integers(-3, 4, size=(4, 64))
    q_idx = _bf16_bits(qi.astype(np.float32))
    scales = np.full(50, np.float16(0.25)).view(np.uint16)
    w = np.array([1, 2, 0.5, 4], np.float32)
    got = oracle.token_scores(codes, scales, q_idx, w)
    for t in range(50):
        ref = sum(float(w[h]) * max(0, int(np.dot(vals[t], qi[h]))) * 0.25 for h in range(4))
        assert got[t] == np.float32(ref)


# ----------------------------------------------------------- block reduce

def test_block_scores_brute_force_with_partial_tail():
    rng = np.random.default_rng(6)
    for L in (1, 3, 4, 5, 8, 13, 64, 67):
        ts = rng.standard_normal(L).astype(np.float32)
        got = oracle.block_scores(ts, 4)
        ref = [max(ts[4 * j:min(4 * j + 4, L)]) for j in range((L + 3) // 4)]
        assert np.array_equal(got, np.array(ref, np.float32))


def test_block_scores_unit_blocks_are_token_scores():
    ts = np.random.default_rng(7).standard_normal(33).astype(np.float32)
    assert np.array_equal(oracle.block_scores(ts, 1), ts)


# -------------------------------------------------------------- selection

def _ref_select(bs, K, forced):
    """Full sort with numpy.lexsort on (-score, index), forced first."""
    n = len(bs)
    if n <= K:
        return np.arange(n)
    f = np.nonzero(forced)[0] if forced is not None else np.zeros(0, int)
    rest = np.setdiff1d(np.arange(n), f)
    order = rest[np.lexsort((rest, -bs[rest].astype(np.float64)))]
    return np.sort(np.concatenate([f, order[:K - len(f)]]))


def test_selection_matches_full_sort_random():
    rng = np.random.default_rng(8)
    for trial in range(200):
        n = int(rng.integers(1, 80))
        K = int(rng.integers(1, 40))
        bs = rng.standard_normal(n).astype(np.float32)
        if trial % 3 == 0:
            bs = rng.integers(0, 4, n).astype(np.float32)          # many ties
        forced = np.zeros(n, np.uint8)
        if trial % 2 == 0:
            forced[rng.choice(n, size=min(n, int(rng.integers(0, 3))), replace=False)] = 1
        if forced.sum() > K and n > K:
            with pytest.raises(ValueError):
                oracle.select_blocks(bs, K, forced)
            continue
        got = oracle.select_blocks(bs, K, forced)
        ref = _ref_select(bs, K, forced)
        assert np.array_equal(got.blocks, ref)
        assert len(got.blocks) == min(n, K)
        assert np.all(np.diff(got.blocks) > 0)
        assert set(np.nonzero(forced)[0]) <= set(got.blocks.tolist()) or n <= K


def test_selection_exhaustive_small_tie_patterns():
    """Every score vector in {0,1,2}^6, every K, with and without a forced block."""
    for scores in itertools.product((0.0, 1.0, 2.0), repeat=6):
        bs = np.array(scores, np.float32)
        for K in range(1, 7):
            for fidx in (None, 0, 5):
                forced = np.zeros(6, np.uint8)
                if fidx is not None:
                    forced[fidx] = 1
                got = oracle.select_blocks(bs, K, forced)
                assert np.array_equal(got.blocks, _ref_select(bs, K, forced))


def test_selection_kth_score_is_last_taken():
    bs = np.array([5, 1, 4, 4, 3, 9], np.float32)
    got = oracle.select_blocks(bs, 3, np.zeros(6, np.uint8))
    assert list(got.blocks) == [0, 2, 5] and got.kth_score == 4.0
    got = oracle.select_blocks(bs, 3, np.array([0, 1, 0, 0, 0, 0], np.uint8))
    assert list(got.blocks) == [0, 1, 5] and got.kth_score == 5.0


def test_forced_mask_sink_and_tail():
    """Sink: the first blocks; tail: every block holding one of the last tokens."""
    m = oracle.forced_mask(4099, 4, sink_blocks=1, tail_tokens=64)
    n_blk = 1025
    assert m.shape == (n_blk,)
    tail_first = (4099 - 64) // 4
    assert np.array_equal(np.nonzero(m)[0], np.r_[0, tail_first:n_blk])
    assert m.sum() == 1 + (n_blk - tail_first)
    assert oracle.forced_mask(10, 4, 0, 64).all()        # tail longer than the context
    assert not oracle.forced_mask(100, 4, 0, 0).any()


def test_tokens_of_blocks_brute_force():
    sel = np.array([0, 3, 4, 9], np.int32)
    L = 38
    ref = [t for j in sel for t in range(4 * j, min(4 * j + 4, L))]
    assert list(oracle.tokens_of_blocks(L, sel, 4)) == ref


# --------------------------------------------------------------- attention

def _rand_pool(rng, n_slots, Hkv=2, Dh=32):
    return _bf16_bits(rng.standard_normal((n_slots, 2 * Hkv * Dh)))


def _sdpa_dense(q_bits, pool_bits, pt, tokens, Hkv, scale):
    """torch scaled_dot_product_attention in float64 on the CPU, GQA by repeat."""
    q = torch.from_numpy(_bf16_values(q_bits))                       # [Hq][Dh]
    rows = torch.from_numpy(_bf16_values(pool_bits[np.asarray(pt)[tokens]]))
    Hq, Dh = q.shape
    K = rows[:, :Hkv * Dh].reshape(-1, Hkv, Dh).permute(1, 0, 2)       # [Hkv][T][Dh]
    V = rows[:, Hkv * Dh:].reshape(-1, Hkv, Dh).permute(1, 0, 2)
    K = K.repeat_interleave(Hq // Hkv, dim=0)
    V = V.repeat_interleave(Hq // Hkv, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q[:, None, :], K, V, scale=scale)
    return o[:, 0, :].numpy()


def test_attention_equals_library_sdpa():
    rng = np.random.default_rng(9)
    Hq, Hkv, Dh = 16, 2, 32
    pool = _rand_pool(rng, 300, Hkv, Dh)
    pt = rng.permutation(300).astype(np.int32)
    tokens = np.sort(rng.choice(300, 77, replace=False))
    q = _bf16_bits(rng.standard_normal((Hq, Dh)) * 2)
    got = oracle.attention(tokens, pt, pool, q, Hkv, 1 / math.sqrt(Dh))
    ref = _sdpa_dense(q, pool, pt, tokens, Hkv, 1 / math.sqrt(Dh))
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)


def test_attention_closed_forms():
    rng = np.random.default_rng(10)
    Hq, Hkv, Dh = 8, 2, 16
    pool = _rand_pool(rng, 50, Hkv, Dh)
    pt = np.arange(50, dtype=np.int32)
    q = _bf16_bits(rng.standard_normal((Hq, Dh)))
    tokens = np.arange(0, 50, 3)
    # constant V -> V
    pc = pool.copy()
    pc[:, Hkv * Dh:] = _bf16_bits(np.full(Hkv * Dh, 1.5))
    assert np.all(oracle.attention(tokens, pt, pc, q, Hkv, 0.25) == np.float32(1.5))
    # q = 0 -> mean of V over the tokens
    got = oracle.attention(tokens, pt, pool, np.zeros_like(q), Hkv, 0.25)
    V = _bf16_values(pool[tokens][:, Hkv * Dh:]).reshape(len(tokens), Hkv, Dh).mean(axis=0)
    for h in range(Hq):
        np.testing.assert_allclose(got[h], V[h // (Hq // Hkv)], rtol=1e-6, atol=1e-7)
    # a single token -> its V
    got = oracle.attention(np.array([7]), pt, pool, q, Hkv, 0.25)
    V7 = _bf16_values(pool[7, Hkv * Dh:]).reshape(Hkv, Dh)
    for h in range(Hq):
        assert np.array_equal(got[h], V7[h // (Hq // Hkv)].astype(np.float32))
    # no tokens -> zeros
    assert not oracle.attention(np.zeros(0, np.int64), pt, pool, q, Hkv, 0.25).any()


def test_attention_page_table_permutation_invariant():
    """Moving rows to other physical slots and updating the page table the same
    way leaves the result bit for bit unchanged (logical order is kept)."""
    rng = np.random.default_rng(11)
    pool = _rand_pool(rng, 120)
    pt = rng.permutation(120).astype(np.int32)
    q = _bf16_bits(rng.standard_normal((16, 32)))
    tokens = np.sort(rng.choice(120, 40, replace=False))
    perm = rng.permutation(120)                    # new slot of old slot s is perm[s]
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    pt2 = perm[pt].astype(np.int32)
    a = oracle.attention(tokens, pt, pool, q, 2, 0.2)
    b = oracle.attention(tokens, pt2, pool2, q, 2, 0.2)
    assert np.array_equal(a, b)


def test_gather_rows_is_page_table_lookup():
    rng = np.random.default_rng(12)
    pool = rng.integers(0, 65535, size=(40, 8)).astype(np.uint16)
    pt = rng.permutation(40).astype(np.int32)
    tokens = np.array([0, 5, 6, 39])
    got = oracle.gather_rows(pool, pt, tokens)
    for p, t in enumerate(tokens):
        assert np.array_equal(got[p], pool[pt[t]])


# ------------------------------------------------------- whole layer

def test_layer_with_budget_covering_context_is_dense_attention():
    """budget >= context selects every block, so the layer is dense softmax
    attention over all tokens (torch SDPA in float64)."""
    rng = np.random.default_rng(13)
    L, Hq, Hkv, Dh = 61, 16, 2, 32
    codes, scales, q_idx = _random_index(rng, L)
    w = rng.uniform(0, 1, 4).astype(np.float32)
    q = _bf16_bits(rng.standard_normal((Hq, Dh)))
    pool = _rand_pool(rng, 90, Hkv, Dh)
    pt = rng.choice(90, L, replace=False).astype(np.int32)
    r = oracle.decode_layer(codes, scales, q_idx, w, q, pt, pool, n_kv_heads=Hkv, budget_tokens=64,
                            sm_scale=1 / math.sqrt(Dh))
    assert list(r.sel) == list(range(16)) and list(r.tokens) == list(range(L))
    ref = _sdpa_dense(q, pool, pt, np.arange(L), Hkv, 1 / math.sqrt(Dh))
    np.testing.assert_allclose(r.out, ref, rtol=1e-6, atol=1e-6)


def test_layer_pipeline_composes_the_steps():
    rng = np.random.default_rng(14)
    L, Hkv, Dh = 203, 2, 32
    codes, scales, q_idx = _random_index(rng, L)
    w = rng.uniform(0, 1, 4).astype(np.float32)
    q = _bf16_bits(rng.standard_normal((16, Dh)))
    pool = _rand_pool(rng, L, Hkv, Dh)
    pt = rng.permutation(L).astype(np.int32)
    r = oracle.decode_layer(codes, scales, q_idx, w, q, pt, pool, n_kv_heads=Hkv, budget_tokens=32,
                            sm_scale=0.2, sink_blocks=1, tail_tokens=9)
    ts = oracle.token_scores(codes, scales, q_idx, w)
    bs = oracle.block_scores(ts)
    fm = oracle.forced_mask(L, 4, 1, 9)
    sel = oracle.select_blocks(bs, 8, fm)
    assert np.array_equal(r.token_scores, ts) and np.array_equal(r.block_scores, bs)
    assert np.array_equal(r.sel, sel.blocks) and len(r.sel) == 8
    assert {0, 48, 49, 50} <= set(r.sel.tolist())          # sink + blocks holding the last 9 tokens
    assert r.tokens[-1] == L - 1
    ref = _sdpa_dense(q, pool, pt, r.tokens, Hkv, 0.2)
    np.testing.assert_allclose(r.out, ref, rtol=1e-6, atol=1e-6)


# ----------------------------------------------------- the pages' numbers

def test_page_byte_facts():
    """Sizes printed on the digest page: 66-byte index keys, 2048-byte KV rows,
    indexer_budget = 2048, 12 QSA layers and 48 MiB moved per decode step."""
    facts = json.load(open(os.path.join(GOLDEN, "page_byte_facts.json")))
    import qsa_synth
    g = qsa_synth.GEOM
    assert g.index_row_bytes == facts["index_bytes_per_token_layer"]
    assert g.row_bytes == facts["kv_bytes_per_token_layer"]
    wl = qsa_synth.WORKLOADS["offload-1m"]
    assert wl.budget == facts["indexer_budget"] and wl.layers == facts["qsa_layers"]
    assert wl.budget * g.row_bytes * wl.layers == facts["selected_bytes_per_step"] == 48 * 2**20


# --------------------------------------------------------------- append step

def test_f16_encoder_matches_numpy():
    """Nearest-value search equals numpy's float16 rounding (a library
    routine): normal, subnormal, exact ties and the overflow edge."""
    rng = np.random.default_rng(21)
    xs = np.concatenate([
        np.abs(rng.standard_normal(300)) * 0.01,
        np.abs(rng.standard_normal(100)) * 1e-6,                 # subnormal range
        (np.arange(1, 60) + 0.5) * 2.0 ** -24,                      # ties between subnormals
        1.0 + (2 * np.arange(40) + 1) * 2.0 ** -11,                 # ties between normals
        [0.0, 65504.0, 65519.0, 65520.0, 70000.0, 2.0 ** -14],
    ]).astype(np.float64)
    for x in xs:
        with np.errstate(over="ignore"):
            want = int(np.float16(x).view(np.uint16))
        assert oracle.encode_f16(x) == want, x


def test_e4m3_encoder_matches_torch_and_saturates():
    """Nearest e4m3 (ties to even) equals torch's float8_e4m3fn rounding
    inside the finite range, including every midpoint between neighbours;
    magnitudes from 448 up clamp to 448 with the sign kept."""
    torch = pytest.importorskip("torch")
    vals = np.array([oracle.decode_e4m3(c) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(22)
    ys = np.concatenate([vals, mids, -mids, rng.uniform(-440, 440, 500), rng.standard_normal(200) * 0.01])
    want = torch.from_numpy(ys.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.encode_e4m3(y) for y in ys.astype(np.float32)], np.uint8)
    assert np.array_equal(got, want)
    for y, code in [(448.0, 0x7E), (449.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE), (464.0, 0x7E)]:
        assert oracle.encode_e4m3(y) == code


def test_quantise_key_properties():
    """Zero key -> zero scale and codes; a key whose largest magnitude is 448
    has scale 1.0 and keeps its representable values exactly; in general the
    largest element lands on +-448 and every element is reconstructed within
    half an e4m3 step."""
    z, s = oracle.quantise_key(np.zeros(64, np.float32))
    assert s == 0 and not z.any()
    vals = np.array([oracle.decode_e4m3(c) for c in range(0x7F)], np.float32)
    x = np.random.default_rng(23).choice(vals, 64).astype(np.float32)
    x[5] = 448.0
    codes, s = oracle.quantise_key(x)
    assert s == 0x3C00
    assert np.array_equal(np.array([oracle.decode_e4m3(c) for c in codes], np.float32), x)
    rng = np.random.default_rng(24)
    for _ in range(20):
        x = (rng.standard_normal(64) * rng.uniform(0.01, 10)).astype(np.float32)
        codes, s = oracle.quantise_key(x)
        sigma = oracle.decode_f16(s)
        assert abs(sigma - np.abs(x).max() / 448) <= 2 ** -11 * sigma
        dec = np.array([oracle.decode_e4m3(c) for c in codes]) * sigma
        assert np.abs(codes & 0x7F).max() == 0x7E
        step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(x) / sigma, 2 ** -6))) - 3), 2 ** -9)
        assert np.all(np.abs(dec - x) <= 0.5 * step * sigma * (1 + 1e-6) + 2 ** -11 * np.abs(x)), x


def test_append_token_reference():
    """The reference append writes the quantised key at row0 + ctx, the row at
    the new slot and the page-table entry, and advances the length."""
    ctx = np.array([3, 0])
    row0 = np.array([0, 10])
    pt = np.full((2, 8), -1, np.int32)
    keys = [np.zeros((20, 64), np.uint8) for _ in range(2)]
    scales = [np.zeros(20, np.uint16) for _ in range(2)]
    pools = [np.zeros((6, 1024), np.uint16) for _ in range(2)]
    rng = np.random.default_rng(25)
    nk = [rng.standard_normal((2, 64)).astype(np.float32) for _ in range(2)]
    nr = [rng.integers(0, 2 ** 16, (2, 1024)).astype(np.uint16) for _ in range(2)]
    out = oracle.append_token(ctx, row0, pt, [4, 1], keys, scales, pools, nk, nr)
    assert list(out) == [4, 1] and pt[0, 3] == 4 and pt[1, 0] == 1
    for l in range(2):
        c, s = oracle.quantise_key(nk[l][0])
        assert np.array_equal(keys[l][3], c) and scales[l][3] == s
        assert np.array_equal(pools[l][4], nr[l][0]) and np.array_equal(pools[l][1], nr[l][1])
        assert not keys[l][4].any() and not pools[l][0].any()


# ---------------------------------------------------------------- hot cache

def test_hot_cache_worked_example():
    """A hand-checked example, H = 4 slots of sequence b = 1 (ids 4..7)."""
    H, b = 4, 1
    hot_map = np.full(20, -1, np.int64)
    owner = np.full(H, -1, np.int64)
    assert oracle.hot_cache_update(hot_map, owner, [2, 5, 9], b, H) == [(2, 0), (5, 1), (9, 2)]
    assert list(owner) == [2, 5, 9, -1] and hot_map[9] == 6
    # 5 hits (slot 1), 3 and 11 miss: slots 0 and 2 are free of hits, so token
    # 2 and token 9 are evicted; token 3 -> slot 0, token 11 -> slot 2
    assert oracle.hot_cache_update(hot_map, owner, [3, 5, 11], b, H) == [(3, 0), (11, 2)]
    assert list(owner) == [3, 5, 11, -1]
    assert hot_map[2] == -1 and hot_map[9] == -1 and hot_map[3] == 4 and hot_map[11] == 6 and hot_map[5] == 5
    # everything cached: no fetch
    assert oracle.hot_cache_update(hot_map, owner, [3, 5], b, H) == []


def test_hot_cache_invariants_random():
    """Over many random steps: map and owner stay inverse to each other, every
    selected token is cached after the update, hits never move, evicted
    tokens were not selected, and the fetch count is the number of selected
    tokens not cached before the step."""
    rng = np.random.default_rng(41)
    n_tok_ctx, H, b = 300, 48, 2
    hot_map = np.full(n_tok_ctx, -1, np.int64)
    owner = np.full(H, -1, np.int64)
    prev = set()
    for step in range(200):
        k = int(rng.integers(0, H + 1))
        keep = [t for t in sorted(prev) if rng.random() < 0.8][:k]
        fresh = rng.choice(n_tok_ctx, k, replace=False).tolist()
        toks = sorted(set(keep) | set(fresh))[:k]
        before_map = hot_map.copy()
        cached_before = {t for t in toks if before_map[t] >= 0}
        fetches = oracle.hot_cache_update(hot_map, owner, toks, b, H)
        assert len(fetches) == len(toks) - len(cached_before)
        assert [t for t, _ in fetches] == sorted(set(toks) - cached_before)
        for t in toks:
            assert hot_map[t] >= 0 and owner[hot_map[t] - b * H] == t
            if t in cached_before:
                assert hot_map[t] == before_map[t]
        for h in range(H):
            if owner[h] >= 0:
                assert hot_map[owner[h]] == b * H + h
        assert (hot_map >= 0).sum() == (owner >= 0).sum()
        evicted = {t for t in range(n_tok_ctx) if before_map[t] >= 0 and hot_map[t] < 0}
        assert not evicted & set(toks)
        prev = set(toks)


# ---------------------------------------------------------------- slot leases

def test_slot_pool_model_worked_example():
    """Ring of 2 slots, 4 tokens: tokens 0 and 1 use the ring; token 2 reuses
    token 0's ring slot after token 0 moves to a body slot, and so on."""
    m = oracle.SlotPoolModel(8)
    a = m.open(2)                                       # ring = slots 0, 1
    assert m.next_token(a) == (0, 0, None)
    assert m.next_token(a) == (1, 0, None)
    assert m.next_token(a) == (0, 0, (0, 0, 2, 0))      # token 0: slot 0 -> body slot 2
    assert m.next_token(a) == (1, 0, (1, 1, 3, 0))
    b = m.open(0)
    assert m.next_token(b) == (4, 0, None)
    assert m.free_slots() == 3
    m.close(a)
    assert m.free_slots() == 7 and m.gen[:5] == [1, 1, 1, 1, 0]
    assert m.next_token(b) == (0, 1, None)              # lowest free slot, new generation


def test_slot_pool_model_reclaims_everything():
    """Random interleavings of opens, appends and closes: no slot is held by
    two leases, and once every lease is closed the free count is back to the
    pool size, with each used slot's generation advanced once per release."""
    rng = np.random.default_rng(51)
    m = oracle.SlotPoolModel(64)
    releases = [0] * 64
    open_ = []
    for _ in range(2000):
        r = rng.random()
        if r < 0.15 or not open_:
            try:
                open_.append(m.open(int(rng.integers(0, 5))))
            except MemoryError:
                pass
        elif r < 0.25:
            lid = open_.pop(int(rng.integers(0, len(open_))))
            held = m.leases[lid]["ring"] + m.leases[lid]["body"]
            for s in held:
                releases[s] += 1
            m.close(lid)
        else:
            try:
                m.next_token(open_[int(rng.integers(0, len(open_)))])
            except MemoryError:
                pass
        held = [s for L in m.leases.values() for s in L["ring"] + L["body"]]
        assert len(held) == len(set(held)) and len(held) + m.free_slots() == 64
    for lid in open_:
        for s in m.leases[lid]["ring"] + m.leases[lid]["body"]:
            releases[s] += 1
        m.close(lid)
    assert m.free_slots() == 64 and m.gen == releases


# ---------------------------------------------------------- multi-query scoring

def test_multi_query_scores_are_causal_single_query_scores():
    """Each query's row equals a brute-force loop over its visible tokens,
    blocks past its position are -inf, and a block cut by the position keeps
    the max over its visible tokens only."""
    rng = np.random.default_rng(81)
    L = 37
    keys = rng.integers(0, 256, (L, 64)).astype(np.uint8)
    keys[(keys & 0x7F) == 0x7F] = 0                     # no NaN codes
    scales = np.float16(rng.uniform(0.01, 1, L)).view(np.uint16)
    q_idx = (torch.from_numpy(rng.standard_normal((3, 4, 64)).astype(np.float32)).to(torch.bfloat16)
             .view(torch.int16).numpy().view(np.uint16))
    w = rng.uniform(0, 1, (3, 4)).astype(np.float32)
    pos = np.array([0, 17, 36])
    got = oracle.multi_block_scores(keys, scales, q_idx, w, pos, 10)
    dec = np.array([[oracle.decode_e4m3(c) for c in row] for row in keys])
    sig = np.array([oracle.decode_f16(s) for s in scales])
    for i, p in enumerate(pos):
        q = np.array([[oracle.decode_bf16(v) for v in row] for row in q_idx[i]])
        s = np.array([sum(w[i, h] * max(0.0, sig[t] * float(q[h] @ dec[t])) for h in range(4)) for t in range(p + 1)])
        for j in range(10):
            lo, hi = 4 * j, min(4 * j + 4, p + 1)
            want = np.float32(s[lo:hi].max()) if lo < hi else -np.inf
            assert got[i, j] == pytest.approx(want, rel=1e-6, abs=1e-30), (i, j)
