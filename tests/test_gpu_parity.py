"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded
synthetic inputs, element by element, plus bit-exact invariances."""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth as S
from qsa_synth import fill
from qsa_synth.device import DeviceInputs

from qsa_testlib import (Unit, check_attention, check_scores, check_selection, oracle_attention_on, oracle_unit,
                          score_scale, unit_inputs)

pytestmark = pytest.mark.gpu

qsa = pytest.importorskip("kv_cache_selection_amd")
G = S.GEOM


def _cfg(wl):
    return qsa.make_config(wl.budget, wl.sink_blocks, wl.tail_tokens, G.sm_scale)


def _batch(di):
    return qsa.make_batch(di.batch, di.max_ctx, di.ctx, di.row0, di.pt, di.pt_stride, di.n_slots, di.n_rows)


def _ws(cfg, B, max_ctx, layers=1, loc=0):
    n = qsa.qsa_workspace_size(cfg, B, max_ctx, layers, loc)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device="cuda"), n


def _u16(t):
    return t.cpu().numpy().view(np.uint16)


# ----------------------------------------------------------------- inputs

def test_fill_matches_host_generator(gpu):
    wl = S.WORKLOADS["tiny-4k"]
    di = DeviceInputs(wl, gpu)
    hi = di.hi
    keys, sig = S.host_index_layer(hi, 0)
    assert np.array_equal(di.keys[0].cpu().numpy(), keys)
    assert np.array_equal(_u16(di.scales[0]), sig)
    slots = np.random.default_rng(0).choice(di.n_slots, 64, replace=False)
    assert np.array_equal(_u16(di.pool[0][torch.from_numpy(slots).to(gpu)]), S.kv_rows(wl.seed, 0, slots))
    wl2 = S.WORKLOADS["batch8-short"]
    di2 = DeviceInputs(wl2, gpu, layers=6)
    L, k2, s2 = unit_inputs(di2.hi, 5, 3)
    r0 = int(di2.hi.lay.row0[3])
    assert np.array_equal(di2.keys[5, r0:r0 + L].cpu().numpy(), k2)
    assert np.array_equal(_u16(di2.scales[5, r0:r0 + L]), s2)


# ---------------------------------------------------------- index scoring

def _score(cfg, B, max_ctx, ctx, row0, keys, scales, q_idx, w, n_rows):
    ts = torch.full((n_rows,), float("nan"), device="cuda")
    bs_stride = (max_ctx + 3) // 4
    bs = torch.full((B, bs_stride), float("nan"), device="cuda")
    bt = qsa.make_batch(B, max_ctx, ctx, row0, n_idx_rows=n_rows)
    qsa.qsa_index_score(cfg, bt, keys, scales, q_idx, w, ts, bs, bs_stride)
    torch.cuda.synchronize()
    return ts.cpu().numpy(), bs.cpu().numpy()


def test_e4m3_decode_all_codes_through_scoring(gpu):
    """Token t carries code c_t in dim 0 and zeros elsewhere; with q = +-e_0,
    w = e_0 and sigma = 1 the score is ReLU(+-decode(c_t)): every finite code,
    compared with torch's e4m3fn decoder."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    L = len(codes)
    keys = np.zeros((L, 64), np.uint8)
    keys[:, 0] = codes
    scales = np.full(L, np.float16(1.0)).view(np.uint16)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    for sign in (1.0, -1.0):
        q_idx = np.zeros((1, 4, 64), np.uint16)
        q_idx[0, 0, 0] = S.f32_to_bf16_bits(np.array([sign], np.float32))[0]
        w = np.array([[1, 0, 0, 0]], np.float32)
        ts, _ = _score(qsa.make_config(256), 1, L, torch.tensor([L], dtype=torch.int32, device=gpu),
                       torch.zeros(1, dtype=torch.int64, device=gpu), torch.from_numpy(keys).to(gpu),
                       torch.from_numpy(scales.view(np.int16)).to(gpu),
                       torch.from_numpy(q_idx.view(np.int16)).to(gpu), torch.from_numpy(w).to(gpu), L)
        assert np.array_equal(ts, np.maximum(0.0, sign * ref).astype(np.float32))


def test_index_score_every_dimension_reaches_its_query_element(gpu):
    """Token t holds 1.0 in dimension t % 64 only and q_h[i] = i + 1 + 64 h
    (exact in bf16): with w = e_h the score must be q_h[t % 64] exactly, so a
    dimension that is dropped, duplicated or permuted on its way from the fp8
    bytes to the matrix cores shows up. (Packing the converted bf16 pairs by
    element once duplicated the low half of every pair.)"""
    L = 256
    keys = np.zeros((L, 64), np.uint8)
    keys[np.arange(L), np.arange(L) % 64] = 0x38
    scales = np.full(L, np.float16(1.0)).view(np.uint16)
    q = np.array([[i + 1 + 64 * h for i in range(64)] for h in range(4)], np.float32)
    q_idx = S.f32_to_bf16_bits(q).reshape(1, 4, 64)
    assert np.array_equal(S.bf16_bits_to_f32(q_idx[0]), q)
    for h in range(4):
        w = np.zeros((1, 4), np.float32)
        w[0, h] = 1.0
        ts, _ = _score(qsa.make_config(64), 1, L, torch.tensor([L], dtype=torch.int32, device=gpu),
                       torch.zeros(1, dtype=torch.int64, device=gpu), torch.from_numpy(keys).to(gpu),
                       torch.from_numpy(scales.view(np.int16)).to(gpu), torch.from_numpy(q_idx.view(np.int16)).to(gpu),
                       torch.from_numpy(w).to(gpu), L)
        assert np.array_equal(ts, q[h, np.arange(L) % 64]), h


@pytest.mark.parametrize("name,layers", [("tiny-4k", 1), ("batch8-short", 2), ("single-38k", 1)])
def test_index_score_parity(gpu, name, layers):
    wl = S.WORKLOADS[name]
    di = DeviceInputs(wl, gpu, layers=layers)
    cfg = _cfg(wl)
    for l in range(layers):
        ts, bs = _score(cfg, di.batch, di.max_ctx, di.ctx, di.row0, di.keys[l], di.scales[l], di.q_idx[l],
                        di.w_idx[l], di.n_rows)
        for b in range(di.batch):
            L, keys, sig = unit_inputs(di.hi, l, b)
            r0 = int(di.hi.lay.row0[b])
            ref_ts = oracle.token_scores(keys, sig, di.hi.q_idx[l, b], di.hi.w[l, b])
            A = score_scale(keys, sig, di.hi.q_idx[l, b], di.hi.w[l, b])
            check_scores(ts[r0:r0 + L], ref_ts, A, "token scores %s l%d b%d" % (name, l, b))
            ref_bs = oracle.block_scores(ref_ts)
            Ab = np.array([A[4 * j:4 * j + 4].max() for j in range(len(ref_bs))])
            check_scores(bs[b, :len(ref_bs)], ref_bs, Ab, "block scores %s l%d b%d" % (name, l, b))
            assert np.isnan(bs[b, len(ref_bs):]).all()       # nothing written past the sequence


def test_index_score_ragged_and_tiny_lengths(gpu):
    """Lengths that are not multiples of 4, 64 or the workgroup tile, and zero."""
    rng = np.random.default_rng(3)
    lens = np.array([1, 3, 4, 5, 63, 64, 65, 255, 257, 1000, 0, 4097], np.int64)
    B = len(lens)
    row0 = np.zeros(B, np.int64)
    row0[1:] = np.cumsum(lens)[:-1]
    n = int(lens.sum())
    keys = rng.integers(0, 256, size=(n, 64)).astype(np.uint8)
    keys[(keys & 0x7F) == 0x7F] = 0x30
    scales = np.float16(rng.uniform(0.001, 0.02, size=n)).view(np.uint16)
    q_idx = S.f32_to_bf16_bits(rng.standard_normal((B, 4, 64)).astype(np.float32))
    w = rng.uniform(0, 1, (B, 4)).astype(np.float32)
    ts, bs = _score(qsa.make_config(64), B, int(lens.max()),
                    torch.from_numpy(lens.astype(np.int32)).to(gpu), torch.from_numpy(row0).to(gpu),
                    torch.from_numpy(keys).to(gpu), torch.from_numpy(scales.view(np.int16)).to(gpu),
                    torch.from_numpy(q_idx.view(np.int16)).to(gpu), torch.from_numpy(w).to(gpu), n)
    for b in range(B):
        L = int(lens[b])
        r0 = int(row0[b])
        k, s = keys[r0:r0 + L], scales[r0:r0 + L]
        ref = oracle.token_scores(k, s, q_idx[b], w[b])
        A = score_scale(k, s, q_idx[b], w[b])
        check_scores(ts[r0:r0 + L], ref, A)
        rb = oracle.block_scores(ref) if L else np.zeros(0, np.float32)
        Ab = np.array([A[4 * j:4 * j + 4].max() for j in range(len(rb))])
        check_scores(bs[b, :len(rb)], rb, Ab)


def test_index_score_integer_exact(gpu):
    """Integer keys/queries, power-of-two scales and weights: all partial sums
    are exact, so the GPU must equal the oracle bit for bit."""
    rng = np.random.default_rng(4)
    L = 3000
    ints = rng.integers(-4, 5, size=(L, 64)).astype(np.float32)
    keys = S.f32_to_e4m3_codes(ints)
    q = rng.integers(-3, 4, size=(1, 4, 64)).astype(np.float32)
    q_idx = S.f32_to_bf16_bits(q)
    scales = np.float16(2.0 ** rng.integers(-6, 2, size=L)).view(np.uint16)
    w = np.array([[0.5, 1.0, 2.0, 0.25]], np.float32)
    ts, bs = _score(qsa.make_config(64), 1, L, torch.tensor([L], dtype=torch.int32, device=gpu),
                    torch.zeros(1, dtype=torch.int64, device=gpu), torch.from_numpy(keys).to(gpu),
                    torch.from_numpy(scales.view(np.int16)).to(gpu), torch.from_numpy(q_idx.view(np.int16)).to(gpu),
                    torch.from_numpy(w).to(gpu), L)
    ref = oracle.token_scores(keys, scales, q_idx[0], w[0])
    assert np.array_equal(ts, ref)
    assert np.array_equal(bs[0], oracle.block_scores(ref))


# --------------------------------------------------------------- selection

def _topk(cfg, bs_rows, lens, K):
    B = len(lens)
    max_ctx = int(max(lens)) if len(lens) else 0
    bs_stride = max(bs_rows.shape[1], 1)
    ctx = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    bt = qsa.make_batch(B, max_ctx, ctx)
    ws, nws = _ws(cfg, B, max_ctx)
    ws.fill_(0xAB)                                  # arbitrary workspace content
    sel = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    ns = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_topk_blocks(cfg, bt, torch.from_numpy(np.ascontiguousarray(bs_rows, np.float32)).cuda(), bs_stride,
                        sel, ns, nt, ws, nws)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), ns.cpu().numpy(), nt.cpu().numpy()


def _check_topk_exact(bs_rows, lens, budget, sink=0, tail=0):
    cfg = qsa.make_config(budget, sink, tail)
    K = budget // 4
    sel, ns, nt = _topk(cfg, bs_rows, lens, K)
    for b, L in enumerate(lens):
        n = (L + 3) // 4
        fm = oracle.forced_mask(L, 4, sink, tail)
        ref = oracle.select_blocks(bs_rows[b, :n], K, fm).blocks
        assert ns[b] == len(ref), (b, ns[b], len(ref))
        assert np.array_equal(sel[b, :ns[b]], ref), (b, L)
        assert np.all(sel[b, ns[b]:] == -1)
        toks = oracle.tokens_of_blocks(L, ref)
        assert nt[b] == len(toks)


# Longest context of the case picks the route: the one-kernel selection with 2
# or 16 scores per thread (up to 8,192 and 65,536 tokens, both ends of the
# second), and the chunk lists with the pool selection past that.
@pytest.mark.parametrize("max_len", [8000, 40000, 65536, 65536 + 1, 262144, 262144 + 4 * 2048 + 1])
def test_topk_exact_random_and_ties(gpu, max_len):
    rng = np.random.default_rng(5 + max_len)
    for trial in range(6):
        lens = rng.integers(1, max_len, size=5)
        lens[4] = max_len
        lens[0] = 4 * 512 + 3          # just over the budget, ragged
        lens[1] = 2048                 # exactly the budget: everything fits
        n_max = (lens.max() + 3) // 4
        if trial % 2:
            bs = rng.integers(0, 50, size=(5, n_max)).astype(np.float32)     # heavy ties
        else:
            bs = rng.standard_normal((5, n_max)).astype(np.float32) * 10
        bs[:, ::7] = -0.0 if trial == 3 else bs[:, ::7]
        _check_topk_exact(bs, lens, 2048, sink=trial % 3, tail=64 if trial >= 3 else 0)


@pytest.mark.parametrize("max_len", [6000, 60000, 262144, 280000])
def test_topk_exact_degenerate_constant_scores(gpu, max_len):
    """All scores equal: every block lands in one histogram bin, so on the
    list route every chunk list is cut short and every chunk is re-read; ties
    break by index."""
    lens = [max_len, 9000, 4 * 512 + 1]
    n_max = (max(lens) + 3) // 4
    bs = np.full((3, n_max), 3.5, np.float32)
    _check_topk_exact(bs, lens, 2048, sink=1)
    bs2 = np.full((3, n_max), 3.5, np.float32)
    bs2[:, 1::2] = np.nextafter(np.float32(3.5), np.float32(10))     # two adjacent values
    _check_topk_exact(bs2, lens, 2048, tail=64)


@pytest.mark.parametrize("max_len", [70001, 262144 + 4 * 2048 + 1])
def test_topk_exact_clustered_scores(gpu, max_len):
    """The answer crowded into a few chunks: their lists (m entries each) are
    wholly chosen, so the pool selection must re-read those chunks; also a
    boost that leaves lists short of the crossing bin, and sequences where
    most of the answer sits in one chunk."""
    rng = np.random.default_rng(7 + max_len)
    lens = [max_len, max_len - 12345, 4 * 512 + 3, 100003]
    n_max = (max(lens) + 3) // 4
    for trial in range(4):
        bs = rng.standard_normal((len(lens), n_max)).astype(np.float32)
        if trial == 0:                          # one dense run of high scores
            bs[:, 5000:7000] += 20.0
        elif trial == 1:                        # several runs in different chunks
            for a in (1000, 9000, 17000):
                bs[:, a:a + 300] += 8.0 + rng.standard_normal((len(lens), 300)).astype(np.float32)
        elif trial == 2:                        # a run of equal top scores inside one chunk
            bs[:, 3000:3900] = 50.0
        else:                                   # rising scores: the last chunks hold the answer
            bs += np.linspace(0.0, 40.0, n_max, dtype=np.float32)[None, :]
        for budget, sink, tail in ((2048, 1, 0), (8192, 0, 64), (64, 0, 0)):
            _check_topk_exact(bs, lens, budget, sink=sink, tail=tail)


@pytest.mark.parametrize("max_len", [40000, 262144 + 4 * 2048 + 1])
def test_topk_exact_infinite_scores(gpu, max_len):
    """Rows as multi-query scoring leaves them for an early query (-inf past
    the visible blocks), +inf and -inf mixed in, and a row of -inf only: on
    the list route, chunks of -inf alone give empty lists, the pool holds
    fewer than r entries, and every incomplete chunk is re-read."""
    rng = np.random.default_rng(11 + max_len)
    lens = [max_len, max_len - 777, 4 * 512 + 3, 50001]
    n_max = (max(lens) + 3) // 4
    bs = rng.standard_normal((len(lens), n_max)).astype(np.float32)
    bs[0, 300:] = -np.inf                                   # visible: the first 300 blocks
    bs[1, rng.random(n_max) < 0.1] = np.inf
    bs[1, rng.random(n_max) < 0.3] = -np.inf
    bs[3, :] = -np.inf
    for budget, sink, tail in ((2048, 1, 0), (2048, 0, 64), (64, 0, 0)):
        _check_topk_exact(bs, lens, budget, sink=sink, tail=tail)


def test_topk_exact_small_budget_many_candidates(gpu):
    rng = np.random.default_rng(6)
    lens = [60000, 123457]
    n_max = (max(lens) + 3) // 4
    bs = np.round(rng.standard_normal((2, n_max)).astype(np.float32) * 4) / 4    # coarse values
    for budget in (4, 64, 8192):
        _check_topk_exact(bs, lens, budget)


# ----------------------------------------------------------------- gather

def test_gather_bit_exact_hbm_and_pinned(gpu):
    wl = S.WORKLOADS["batch8-short"]
    di = DeviceInputs(wl, gpu, layers=1)
    cfg = _cfg(wl)
    K = wl.budget // 4
    sel = np.full((di.batch, K), -1, np.int32)
    ns = np.zeros(di.batch, np.int32)
    rng = np.random.default_rng(7)
    toks_ref = []
    for b in range(di.batch):
        L = int(di.hi.lay.ctx[b])
        n = (L + 3) // 4
        k = int(rng.integers(1, min(K, n) + 1)) if b else min(K, n)
        s = np.sort(rng.choice(n, k, replace=False)).astype(np.int32)
        if b == 1 and (n - 1) not in s:
            s[-1] = n - 1                                    # include the partial last block
            s = np.unique(s)
        sel[b, :len(s)] = s
        ns[b] = len(s)
        toks_ref.append(oracle.tokens_of_blocks(L, s))
    out = torch.full((di.batch, wl.budget, G.row_elems), 0x5A5A, dtype=torch.int16, device=gpu)
    nt = torch.zeros(di.batch, dtype=torch.int32, device=gpu)
    sel_d, ns_d = torch.from_numpy(sel).to(gpu), torch.from_numpy(ns).to(gpu)
    qsa.qsa_gather_kv(cfg, _batch(di), sel_d, ns_d, di.pool[0], qsa.QSA_KV_DEVICE, out, nt)
    torch.cuda.synchronize()
    got = _u16(out)
    pool0 = _u16(di.pool[0])
    for b in range(di.batch):
        toks = toks_ref[b]
        assert int(nt[b]) == len(toks)
        ref = oracle.gather_rows(pool0, di.hi.lay.pt[b], toks)
        assert np.array_equal(got[b, :len(toks)], ref)
        assert np.all(got[b, len(toks):] == 0x5A5A)          # untouched past n_tok
    # the same rows from pinned host memory over PCIe
    host_pool = torch.empty_like(di.pool[0], device="cpu").pin_memory()
    host_pool.copy_(di.pool[0])
    out2 = torch.full_like(out, 0x5A5A)
    qsa.qsa_gather_kv(cfg, _batch(di), sel_d, ns_d, host_pool, qsa.QSA_KV_HOST_PINNED, out2, nt)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


# --------------------------------------------------------------- attention

def _decode(cfg, q, kv, nt):
    B = q.shape[0]
    ws, nws = _ws(cfg, B, 0)
    out = torch.full((B, 16, 256), float("nan"), device="cuda")
    qsa.qsa_sparse_decode(cfg, B, q, kv, nt, out, ws, nws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_sparse_decode_parity_and_closed_forms(gpu):
    rng = np.random.default_rng(8)
    budget = 2048
    cfg = qsa.make_config(budget)
    B = 5
    ntok = np.array([2048, 1, 0, 1000, 65], np.int32)
    kv = S.f32_to_bf16_bits(rng.standard_normal((B, budget, G.row_elems)).astype(np.float32))
    q = S.f32_to_bf16_bits(rng.standard_normal((B, 16, 256)).astype(np.float32))
    got = _decode(cfg, torch.from_numpy(q.view(np.int16)).cuda(), torch.from_numpy(kv.view(np.int16)).cuda(),
                  torch.from_numpy(ntok).cuda())
    for b in range(B):
        ref = oracle.attention(np.arange(ntok[b]), None, kv[b], q[b], 2, G.sm_scale)
        check_attention(got[b], ref, "sequence %d" % b)
    assert np.all(got[2] == 0)                                      # no tokens -> zeros
    v1 = S.bf16_bits_to_f32(kv[1, 0, 512:]).reshape(2, 256)         # one token -> its V
    assert np.array_equal(got[1], np.repeat(v1, 8, axis=0))
    # constant V -> V, up to fp32 rounding of the weighted sum and its normaliser
    kvc = kv.copy()
    kvc[:, :, 512:] = S.f32_to_bf16_bits(np.float32(-0.75))
    got = _decode(cfg, torch.from_numpy(q.view(np.int16)).cuda(), torch.from_numpy(kvc.view(np.int16)).cuda(),
                  torch.from_numpy(ntok).cuda())
    assert np.abs(got[ntok > 0] + 0.75).max() <= 4 * np.spacing(np.float32(0.75))


@pytest.mark.parametrize("budget", [640, 1500, 2600])
def test_sparse_decode_split_counts(gpu, budget):
    """Split counts that are not a multiple of the merge's batch of splits:
    10, 24 and 41 splits of 64 tokens (or 5, 12 and 21 of 128). The merge
    loads past the last split are clamped and masked, and 41 splits take a
    second batch that continues the online rescale. Full, ragged and half
    sequences against the oracle."""
    rng = np.random.default_rng(budget)
    cfg = qsa.make_config(budget)
    B = 3
    ntok = np.array([budget, budget - 3, budget // 2 + 1], np.int32)
    kv = S.f32_to_bf16_bits(rng.standard_normal((B, budget, G.row_elems)).astype(np.float32))
    q = S.f32_to_bf16_bits(rng.standard_normal((B, 16, 256)).astype(np.float32))
    got = _decode(cfg, torch.from_numpy(q.view(np.int16)).cuda(), torch.from_numpy(kv.view(np.int16)).cuda(),
                  torch.from_numpy(ntok).cuda())
    for b in range(B):
        ref = oracle.attention(np.arange(ntok[b]), None, kv[b], q[b], 2, G.sm_scale)
        check_attention(got[b], ref, "budget %d, sequence %d" % (budget, b))


# ------------------------------------------------------------- whole step

def _step(di, loc=None, n_side=2):
    wl = di.wl
    cfg = _cfg(wl)
    K = wl.budget // 4
    L = di.n_layers
    loc = (qsa.QSA_KV_HOST_PINNED if di.kv_host else qsa.QSA_KV_DEVICE) if loc is None else loc
    sel = torch.full((L, di.batch, K), -7, dtype=torch.int32, device="cuda")
    ns = torch.zeros((L, di.batch), dtype=torch.int32, device="cuda")
    layers = [qsa.make_layer(di.keys[l], di.scales[l], di.q_idx[l], di.w_idx[l], di.q[l], di.pool[l], di.out[l],
                             None, sel[l], ns[l]) for l in range(L)]
    ws, nws = _ws(cfg, di.batch, di.max_ctx, L, loc)
    side = [torch.cuda.Stream() for _ in range(n_side)]
    ev = qsa.StepEvents(L, n_side) if n_side else None
    qsa.qsa_decode_step(cfg, _batch(di), layers, loc, ws, nws, torch.cuda.current_stream(), side, events=ev)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), ns.cpu().numpy(), di.out.cpu().numpy()


def _check_step_units(di, sel, ns, out, units):
    excused = 0
    for (l, b) in units:
        u = oracle_unit(di.hi, l, b)
        gsel = sel[l, b, :ns[l, b]]
        excused += check_selection(gsel, u)
        toks = u.tokens if np.array_equal(gsel, u.sel) else oracle.tokens_of_blocks(u.L, gsel)
        ref = oracle_attention_on(di.hi, l, b, toks)
        check_attention(out[l, b], ref, "unit %s" % ((l, b),))
    return excused


# The longest context picks the selection route: the one-kernel selection
# (65,536 tokens) or the chunk lists (70,001).
@pytest.mark.parametrize("longest", [65536, 70001])
def test_decode_step_edge_lengths(gpu, longest):
    """A batch of edge lengths through the whole step: an empty sequence, one
    and three tokens (a partial first block, forced as the sink), exactly the
    budget (everything fits), just over it with partial last blocks (L mod 4
    = 1 and 3), a mid length and the longest; with a sink block and a 64-token
    tail ring. Every schedule and the pinned-host pool give the same bits, and
    every (layer, sequence) matches the oracle; the empty sequence attends to
    nothing and returns zeros."""
    wl = S.Workload("edge-lengths", 8, (0, 1, 3, 2048, 2049, 2051, 9000, longest), 2, 2048, sink_blocks=1,
                    tail_tokens=64, planted=8, seed=11)
    di = DeviceInputs(wl, gpu)
    sel, ns, out = _step(di, n_side=0)
    for n_side in (1, 2):
        sel2, ns2, out2 = _step(di, n_side=n_side)
        assert np.array_equal(sel, sel2) and np.array_equal(ns, ns2) and np.array_equal(out, out2), n_side
    dh = DeviceInputs(wl, gpu, kv_host=True, hi=di.hi)
    sel3, ns3, out3 = _step(dh, n_side=1)
    assert np.array_equal(sel, sel3) and np.array_equal(out, out3)
    assert np.all(ns[:, 0] == 0) and np.all(out[:, 0] == 0.0)
    assert np.all(ns[:, 3] == 512)                  # 2048 tokens: all 512 blocks fit
    _check_step_units(di, sel, ns, out, [(l, b) for l in range(wl.layers) for b in range(wl.batch)])


@pytest.mark.parametrize("name,layers", [("tiny-4k", 1), ("batch8-short", 3), ("single-38k", 2)])
def test_decode_step_parity(gpu, name, layers):
    di = DeviceInputs(S.WORKLOADS[name], gpu, layers=layers)
    sel, ns, out = _step(di)
    units = [(l, b) for l in range(layers) for b in range(di.batch)]
    _check_step_units(di, sel, ns, out, units)
    # planted blocks are recovered (a sanity property of the synthetic data)
    for (l, b) in units:
        planted = di.hi.lay.planted[(l, b)]
        assert set(planted.tolist()) <= set(sel[l, b, :ns[l, b]].tolist())


def test_decode_step_deterministic_and_offload_bit_exact(gpu):
    """Every schedule gives the same bits: one stream, one to three side
    streams, and the offload path (pool in pinned host memory, gather over
    PCIe on a side stream), which must match the HBM path that reads the rows
    in place through the page table."""
    wl = S.WORKLOADS["batch8-short"]
    di = DeviceInputs(wl, gpu, layers=5)
    sel1, ns1, out1 = _step(di)
    for n_side in (0, 1, 3):
        sel2, ns2, out2 = _step(di, n_side=n_side)
        assert np.array_equal(out1, out2) and np.array_equal(sel1, sel2), n_side
    dh = DeviceInputs(wl, gpu, layers=5, kv_host=True, hi=di.hi)
    for n_side in (1, 0, 2):
        sel3, ns3, out3 = _step(dh, n_side=n_side)
        assert np.array_equal(sel1, sel3), n_side
        assert np.array_equal(out1, out3), n_side


def _list_geom(B, max_ctx, K):
    """(blocks per scoring chunk, m, cap) of the chunk lists, the rule the
    library applies (score chunk: 512 tokens, doubled while the call keeps
    512 workgroups per layer, up to 8192; m about three times a chunk's share
    of the budget, at least 8 while all lists fit 8192 slots, else 4)."""
    chunk = 512
    while chunk < 8192 and B * ((max_ctx + 2 * chunk - 1) // (2 * chunk)) >= 512:
        chunk *= 2
    cb = chunk // 4
    n_chunks = ((max_ctx + 3) // 4 + cb - 1) // cb
    floor = 8 if n_chunks * 16 <= 8192 else 4
    m = min(max((3 * K + n_chunks - 1) // n_chunks, floor), 64)
    return cb, m, 2 * m


def test_decode_step_scores_re_read_chunks_again(gpu):
    """In the decode step the scan keeps a chunk's block scores only when the
    chunk's list was cut short by a crowded bin; a chunk that the selection
    must re-read otherwise is scored again from the index. Here a run of 16
    chunks per sequence and layer holds keys along the query with scales that
    rise over four octaves in every 512 tokens: each run chunk holds about 32
    of the answer's blocks, spread over some 32 bins, so its list (about m
    entries) is not cut short, is wholly chosen, and the chunk is re-read and
    scored again. Two layers (runs in different places), a sink block and a
    64-token tail; one stream (per-layer launches), a side stream (one launch
    per kernel for both layers) and the pinned-host pipeline. Every schedule
    must give the same bits, and each selection must equal the exact top-K of
    the block scores that the standalone scoring call computes (the same
    arithmetic) and match the oracle's within near ties."""
    from test_list_route_model import chunk_list, list_route, order_keys
    rng = np.random.default_rng(17)
    lens = np.array([100000, 70001], np.int64)
    B, NL = len(lens), 2
    row0 = np.array([0, int(lens[0])], np.int64)
    n = int(lens.sum())
    budget, K, sink, tail = 2048, 512, 1, 64
    runs = {(0, 0): 20000, (0, 1): 30720, (1, 0): 61440, (1, 1): 4096}   # (layer, b): first token of the run
    keys = np.empty((NL, n, 64), np.uint8)
    scales = np.empty((NL, n), np.uint16)
    q_idx = np.empty((NL, B, 4, 64), np.uint16)
    w = rng.uniform(0.5, 1.0, (NL, B, 4)).astype(np.float32)
    for l in range(NL):
        kl = rng.integers(0, 256, size=(n, 64)).astype(np.uint8)
        kl[(kl & 0x7F) == 0x7F] = 0x30
        sl = np.float16(rng.uniform(0.001, 0.02, size=n))
        v = rng.standard_normal((B, 64)).astype(np.float32)
        q_idx[l] = S.f32_to_bf16_bits(np.repeat(v[:, None, :], 4, axis=1))
        for b in range(B):
            vb = S.bf16_bits_to_f32(q_idx[l, b, 0])
            code = S.f32_to_e4m3_codes(vb / np.abs(vb).max() * 448.0)
            t0 = int(row0[b]) + runs[(l, b)]
            for c in range(16):
                kl[t0 + 512 * c:t0 + 512 * (c + 1)] = code
                sl[t0 + 512 * c:t0 + 512 * (c + 1)] = np.float16(
                    1e-3 * np.exp2(4.0 * np.arange(512) / 512 + 0.013 * c))
        keys[l], scales[l] = kl, sl.view(np.uint16)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu)
    max_ctx = int(lens.max())
    ctx, r0d = d(lens.astype(np.int32)), d(row0)
    keys_d, scales_d = d(keys), d(scales.view(np.int16))
    q_idx_d, w_d = d(q_idx.view(np.int16)), d(w)
    cb, m, cap = _list_geom(B, max_ctx, K)
    bs = []                                         # the GPU's own block scores, from the standalone call
    for l in range(NL):
        _, bl = _score(qsa.make_config(budget, sink, tail), B, max_ctx, ctx, r0d, keys_d[l], scales_d[l],
                       q_idx_d[l], w_d[l], n)
        bs.append(bl)
        for b in range(B):                          # the construction does what it is for
            nb = (int(lens[b]) + 3) // 4
            tail_first = max(int(lens[b]) - tail, 0) // 4
            _, n_needy = list_route(bl[b, :nb], K, sink, tail_first, cb, m, cap)
            assert n_needy >= 8, (l, b, n_needy)
            j0 = runs[(l, b)] // 4
            theta, complete, comps = chunk_list(order_keys(bl[b, j0:j0 + cb]), np.arange(j0, j0 + cb), m, cap)
            assert len(comps) >= m and not complete     # a full list, not cut short
    n_slots = n
    pool = torch.randn((NL, n_slots, 1024), dtype=torch.bfloat16, device=gpu).view(torch.int16)
    pool_h = torch.empty((NL, n_slots, 1024), dtype=torch.int16, pin_memory=True)
    pool_h.copy_(pool)
    pt = np.stack([np.arange(max_ctx) + row0[b] for b in range(B)])
    pt = d(np.where(pt < n, pt, 0).astype(np.int32))
    q = torch.randn((NL, B, 16, 256), dtype=torch.bfloat16, device=gpu).view(torch.int16)
    cfg = qsa.make_config(budget, sink, tail)
    bt = qsa.make_batch(B, max_ctx, ctx, r0d, pt, int(pt.shape[1]), n_slots, n)
    got = []
    for loc, n_side in ((qsa.QSA_KV_DEVICE, 0), (qsa.QSA_KV_DEVICE, 1), (qsa.QSA_KV_HOST_PINNED, 1)):
        ws, nws = _ws(cfg, B, max_ctx, NL, loc)
        ws.fill_(0xAB)                              # no stale block scores to find
        sel = torch.full((NL, B, K), -7, dtype=torch.int32, device=gpu)
        ns = torch.zeros((NL, B), dtype=torch.int32, device=gpu)
        out = torch.zeros((NL, B, 16, 256), dtype=torch.float32, device=gpu)
        pl = pool if loc == qsa.QSA_KV_DEVICE else pool_h
        lay = [qsa.make_layer(keys_d[l], scales_d[l], q_idx_d[l], w_d[l], q[l], pl[l], out[l], None, sel[l], ns[l])
               for l in range(NL)]
        side = [torch.cuda.Stream() for _ in range(n_side)]
        ev = qsa.StepEvents(NL, n_side) if n_side else None
        qsa.qsa_decode_step(cfg, bt, lay, loc, ws, nws, torch.cuda.current_stream(), side, events=ev)
        torch.cuda.synchronize()
        got.append((sel.cpu().numpy(), ns.cpu().numpy(), out.cpu().numpy()))
    for other in got[1:]:
        for a, b_ in zip(got[0], other):
            assert np.array_equal(a, b_)
    sel, ns, _ = got[0]
    for l in range(NL):
        for b in range(B):
            L = int(lens[b])
            nb = (L + 3) // 4
            fm = oracle.forced_mask(L, 4, sink, tail)
            exact = oracle.select_blocks(bs[l][b, :nb], K, fm).blocks   # exact top-K of the GPU's block scores
            assert ns[l, b] == len(exact)
            assert np.array_equal(sel[l, b, :ns[l, b]], exact), (l, b)
            k, s = keys[l, row0[b]:row0[b] + L], scales[l, row0[b]:row0[b] + L]
            ref_bs = oracle.block_scores(oracle.token_scores(k, s, q_idx[l, b], w[l, b]))
            osel = oracle.select_blocks(ref_bs, K, fm)
            check_selection(sel[l, b, :ns[l, b]], Unit(L, None, None, None, None, None, None, None, ref_bs, fm,
                                                       osel.blocks, osel.kth_score, None))


def test_decode_step_offload_reuses_one_event_set(gpu):
    """One event set and one side stream serve several pinned-host pipeline
    calls in a row, as in a decode loop: the set's signal carries a larger
    value at every hand-over. The queries change between the calls, so a
    gather that started before its group's selection had been written would
    copy the previous call's rows; every call must give the one-stream bits
    of its own inputs."""
    wl = S.WORKLOADS["batch8-short"]
    dh = DeviceInputs(wl, gpu, layers=5, kv_host=True)
    perm = torch.roll(torch.arange(dh.batch, device="cuda"), 1)
    states = [(dh.q_idx.clone(), dh.q.clone()), (dh.q_idx[:, perm].clone(), dh.q[:, perm].clone())]
    ref = []
    for qi, q in states:
        dh.q_idx.copy_(qi)
        dh.q.copy_(q)
        ref.append(_step(dh, n_side=0))
    assert not np.array_equal(ref[0][0], ref[1][0])
    cfg = _cfg(wl)
    K = wl.budget // 4
    L = dh.n_layers
    ws, nws = _ws(cfg, dh.batch, dh.max_ctx, L, qsa.QSA_KV_HOST_PINNED)
    side = [torch.cuda.Stream()]
    ev = qsa.StepEvents(L, 1)
    for i in (0, 1, 1, 0, 1, 0):
        dh.q_idx.copy_(states[i][0])
        dh.q.copy_(states[i][1])
        sel = torch.full((L, dh.batch, K), -7, dtype=torch.int32, device="cuda")
        ns = torch.zeros((L, dh.batch), dtype=torch.int32, device="cuda")
        layers = [qsa.make_layer(dh.keys[l], dh.scales[l], dh.q_idx[l], dh.w_idx[l], dh.q[l], dh.pool[l],
                                 dh.out[l], None, sel[l], ns[l]) for l in range(L)]
        qsa.qsa_decode_step(cfg, _batch(dh), layers, qsa.QSA_KV_HOST_PINNED, ws, nws,
                            torch.cuda.current_stream(), side, events=ev)
        torch.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), ref[i][0]), i
        assert np.array_equal(ns.cpu().numpy(), ref[i][1]), i
        assert np.array_equal(dh.out.cpu().numpy(), ref[i][2]), i


def test_decode_step_more_layers_than_one_group(gpu):
    """The overlapped schedules scan, select and attend up to 16 layers per
    launch; 18 layers take two groups (16 + 2), and every schedule, with the
    pool in HBM or in pinned host memory, must still give the one-stream
    bits, which match the oracle."""
    wl = S.Workload("groups-18", 2, (3001, 1800), 18, 256, planted=4, seed=21)
    di = DeviceInputs(wl, gpu)
    sel0, ns0, out0 = _step(di, n_side=0)
    for n_side in (1, 2, 3):
        sel, ns, out = _step(di, n_side=n_side)
        assert np.array_equal(sel0, sel) and np.array_equal(ns0, ns), n_side
        assert np.array_equal(out0, out), n_side
    _check_step_units(di, sel0, ns0, out0, [(0, 0), (15, 1), (16, 0), (17, 1)])
    # the pinned-host pool path groups the same way (scan, select, gather, attend)
    dh = DeviceInputs(wl, gpu, kv_host=True, hi=di.hi)
    for n_side in (0, 1):
        sel, ns, out = _step(dh, n_side=n_side)
        assert np.array_equal(sel0, sel) and np.array_equal(ns0, ns), n_side
        assert np.array_equal(out0, out), n_side


def test_decode_step_page_table_permutation_invariant(gpu):
    """Moving every row to another slot and rewriting the page table the same
    way leaves the output bit for bit unchanged."""
    wl = S.WORKLOADS["tiny-4k"]
    di = DeviceInputs(wl, gpu)
    _, _, out1 = _step(di)
    perm = torch.from_numpy(np.random.default_rng(9).permutation(di.n_slots)).to(gpu)
    pool2 = torch.empty_like(di.pool)
    pool2[:, perm] = di.pool
    di.pool = pool2
    di.pt = torch.where(di.pt >= 0, perm[di.pt.clamp(min=0).long()].int(), di.pt)
    _, _, out2 = _step(di)
    assert np.array_equal(out1, out2)


def test_decode_step_per_layer_page_table(gpu):
    """A layer may bring its own page table (qsa_layer_t.page_table): moving
    layer 1's rows to other slots of its pool and giving that layer the
    rewritten table leaves every output bit for bit unchanged, on one stream,
    in the grouped HBM schedule and on the pinned-host path."""
    wl = S.WORKLOADS["batch8-short"]
    di = DeviceInputs(wl, gpu, layers=3)
    K = wl.budget // 4
    L = di.n_layers
    perm = torch.from_numpy(np.random.default_rng(11).permutation(di.n_slots)).to(gpu)
    pool1 = torch.empty_like(di.pool[1])
    pool1[perm] = di.pool[1]
    pt1 = torch.where(di.pt >= 0, perm[di.pt.clamp(min=0).long()].int(), di.pt)
    for kv_host in (False, True):
        d = di if not kv_host else DeviceInputs(wl, gpu, layers=3, kv_host=True, hi=di.hi)
        loc = qsa.QSA_KV_HOST_PINNED if kv_host else qsa.QSA_KV_DEVICE
        p1 = pool1 if not kv_host else pool1.cpu().pin_memory()
        for n_side in (0, 1):
            outs = []
            for own_table in (False, True):
                sel = torch.full((L, d.batch, K), -7, dtype=torch.int32, device="cuda")
                ns = torch.zeros((L, d.batch), dtype=torch.int32, device="cuda")
                d.out.zero_()
                layers = [qsa.make_layer(d.keys[l], d.scales[l], d.q_idx[l], d.w_idx[l], d.q[l],
                                         p1 if (own_table and l == 1) else d.pool[l], d.out[l],
                                         pt1 if (own_table and l == 1) else None, sel[l], ns[l]) for l in range(L)]
                cfg = _cfg(wl)
                ws, nws = _ws(cfg, d.batch, d.max_ctx, L, loc)
                side = [torch.cuda.Stream() for _ in range(n_side)]
                ev = qsa.StepEvents(L, n_side) if n_side else None
                qsa.qsa_decode_step(cfg, _batch(d), layers, loc, ws, nws, torch.cuda.current_stream(), side,
                                    events=ev)
                torch.cuda.synchronize()
                outs.append((sel.cpu().numpy(), d.out.cpu().numpy()))
            assert np.array_equal(outs[0][0], outs[1][0]), (kv_host, n_side)
            assert np.array_equal(outs[0][1], outs[1][1]), (kv_host, n_side)


def test_decode_step_budget_covers_context_is_dense(gpu):
    """With the budget above the context every block is selected and the step
    is dense softmax attention over all tokens."""
    wl = S.Workload("dense", 2, (1501, 2048), 1, 2048, seed=11)
    di = DeviceInputs(wl, gpu)
    sel, ns, out = _step(di)
    for b in range(2):
        L = int(di.hi.lay.ctx[b])
        assert ns[0, b] == (L + 3) // 4
        ref = oracle_attention_on(di.hi, 0, b, np.arange(L))
        check_attention(out[0, b], ref, "dense %d" % b)


def test_decode_step_reports_bad_entries(gpu):
    """Device-side values that break the contract are clamped (every read stays
    in bounds) and reported in the workspace's flags word: a clean step
    leaves it 0; a page-table entry outside the pool on a token that every
    selection takes (the tail ring's last token) raises QSA_FLAG_BAD_SLOT,
    from the fused attention (HBM pool) and from the gather (pinned-host
    pool); a context length above max_ctx raises QSA_FLAG_BAD_CTX_LEN; index
    rows past the index buffer raise QSA_FLAG_BAD_INDEX_ROWS. The next clean
    call clears the word."""
    wl = S.WORKLOADS["batch8-short"]
    di = DeviceInputs(wl, gpu, layers=2)
    dh = DeviceInputs(wl, gpu, layers=2, kv_host=True, hi=di.hi)
    cfg = _cfg(wl)
    K = wl.budget // 4
    flags = torch.full((1,), -1, dtype=torch.int32, device=gpu)

    def run(d, loc, pt=None, ctx=None, n_rows=None, n_side=0):
        sel = torch.full((2, d.batch, K), -7, dtype=torch.int32, device=gpu)
        ns = torch.zeros((2, d.batch), dtype=torch.int32, device=gpu)
        layers = [qsa.make_layer(d.keys[l], d.scales[l], d.q_idx[l], d.w_idx[l], d.q[l], d.pool[l], d.out[l],
                                 None, sel[l], ns[l]) for l in range(2)]
        bt = qsa.make_batch(d.batch, d.max_ctx, d.ctx if ctx is None else ctx, d.row0, d.pt if pt is None else pt,
                            d.pt_stride, d.n_slots, d.n_rows if n_rows is None else n_rows)
        ws, nws = _ws(cfg, d.batch, d.max_ctx, 2, loc)
        ws.fill_(0x77)
        side = [torch.cuda.Stream() for _ in range(n_side)]
        ev = qsa.StepEvents(2, n_side) if n_side else None
        qsa.qsa_decode_step(cfg, bt, layers, loc, ws, nws, torch.cuda.current_stream(), side, events=ev)
        qsa.qsa_read_flags(ws, flags)
        torch.cuda.synchronize()
        return int(flags[0]), ns.cpu().numpy()

    hbm, pin = qsa.QSA_KV_DEVICE, qsa.QSA_KV_HOST_PINNED
    assert run(di, hbm)[0] == 0 and run(dh, pin)[0] == 0
    L3 = int(di.hi.lay.ctx[3])
    bad_pt = di.pt.clone()
    bad_pt[3, L3 - 1] = di.n_slots + 5
    for d, loc in ((di, hbm), (dh, pin)):
        for n_side in (0, 1):
            assert run(d, loc, pt=bad_pt, n_side=n_side)[0] == qsa.QSA_FLAG_BAD_SLOT, (loc, n_side)
    neg_pt = di.pt.clone()
    neg_pt[3, L3 - 1] = -3
    assert run(di, hbm, pt=neg_pt)[0] == qsa.QSA_FLAG_BAD_SLOT
    # the longest sequence claims one token more than max_ctx: clamped back to
    # its own length, so only the length is reported
    ctx = di.ctx.clone()
    ctx[int(np.argmax(di.hi.lay.ctx))] = di.max_ctx + 1
    assert run(di, hbm, ctx=ctx)[0] == qsa.QSA_FLAG_BAD_CTX_LEN
    f, ns = run(di, hbm, n_rows=di.n_rows - 1)           # the last sequence's rows run past the buffer
    assert f == qsa.QSA_FLAG_BAD_INDEX_ROWS
    assert np.all(ns[:, -1] == 0) and np.all(ns[:, 0] > 0)
    assert run(di, hbm)[0] == 0
