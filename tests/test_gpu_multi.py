"""Parity of multi-query scoring (qsa_index_score_multi) with the oracle's
causal per-query block scores, for every supported query count, with query
positions at the start, in the middle, on block boundaries and at the end,
and at the full batch8-256k size on sampled queries."""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth as S
from qsa_synth import host as SH
from qsa_synth.device import DeviceInputs

from qsa_testlib import check_scores, score_scale

pytestmark = pytest.mark.gpu

qsa = pytest.importorskip("kv_cache_selection_amd")
G = S.GEOM


def _run(di, Q, pos, rng, layer=0):
    B = di.batch
    q_idx = S.f32_to_bf16_bits(rng.standard_normal((B, Q, G.idx_heads, G.idx_dim)).astype(np.float32))
    w = rng.uniform(0, 1, (B, Q, G.idx_heads)).astype(np.float32)
    nb = (di.max_ctx + 3) // 4
    out = torch.full((B, Q, nb + 3), 7.0, device="cuda")          # 7.0 marks entries that must stay untouched
    cfg = qsa.make_config(2048)
    bt = qsa.make_batch(B, di.max_ctx, di.ctx, di.row0, di.pt, di.pt_stride, di.n_slots, di.n_rows)
    qsa.qsa_index_score_multi(cfg, bt, Q, di.keys[layer], di.scales[layer],
                              torch.from_numpy(q_idx.view(np.int16)).cuda(), torch.from_numpy(w).cuda(),
                              torch.from_numpy(np.asarray(pos, np.int32)).cuda(), out, nb + 3)
    torch.cuda.synchronize()
    return q_idx, w, out.cpu().numpy()


def _check(di, layer, b, keys, sig, q_idx, w, pos, got):
    L = int(di.hi.lay.ctx[b])
    nblk = (L + 3) // 4
    ref = oracle.multi_block_scores(keys, sig, q_idx, w, pos, nblk)
    for i in range(len(pos)):
        inf_ref = np.isneginf(ref[i])
        assert np.array_equal(np.isneginf(got[i, :nblk]), inf_ref), i
        A = score_scale(keys, sig, q_idx[i], w[i])
        A = np.pad(A, (0, 4 * nblk - L)).reshape(nblk, 4).max(axis=1)
        ok = ~inf_ref
        check_scores(got[i, :nblk][ok], ref[i][ok], A[ok], "query %d" % i)
        assert np.all(got[i, nblk:] == 7.0)


@pytest.mark.parametrize("Q", [4, 16, 64])
def test_multi_query_scores(gpu, Q):
    wl = S.Workload("multi", 2, (5001, 3000), 1, 2048, seed=13)
    di = DeviceInputs(wl, gpu)
    rng = np.random.default_rng(90 + Q)
    pos = np.zeros((di.batch, Q), np.int64)
    for b in range(di.batch):
        L = int(di.hi.lay.ctx[b])
        special = [0, 1, 3, 4, 255, 256, L // 2, L - 1, L + 5]        # L + 5: sees everything
        p = list(range(L - Q, L))                                       # a chunk at the end
        p[:len(special)] = special
        pos[b] = p[:Q]
    q_idx, w, got = _run(di, Q, pos, rng)
    for b in range(di.batch):
        L = int(di.hi.lay.ctx[b])
        keys, sig = SH.index_keys(wl.seed, 0, b, 0, L, di.hi.lay.planted[(0, b)], di.hi.u[0, b])
        _check(di, 0, b, keys, sig, q_idx[b], w[b], np.minimum(pos[b], L - 1), got[b])


@pytest.mark.slow
def test_multi_query_scores_full_size_sampled(gpu):
    """64 queries per sequence over batch8-256k's index, the chunk at the end of
    each sequence; three queries of two sequences checked in full."""
    wl = S.WORKLOADS["batch8-256k"]
    di = DeviceInputs(wl, gpu, layers=1)
    rng = np.random.default_rng(99)
    L = int(di.hi.lay.ctx[0])
    pos = np.tile(np.arange(L - 64, L), (di.batch, 1))
    q_idx, w, got = _run(di, 64, pos, rng)
    for b in (0, 5):
        keys, sig = SH.index_keys(wl.seed, 0, b, 0, L, di.hi.lay.planted[(0, b)], di.hi.u[0, b])
        sub = [0, 31, 63]
        _check(di, 0, b, keys, sig, q_idx[b, sub], w[b, sub], pos[b, sub], got[b, sub])
