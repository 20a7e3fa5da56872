"""Parity of the hot row cache (qsa_hot_cache_t in qsa_decode_step, pinned-host
pools): over several decode steps with drifting queries, the cache mapping
must equal the oracle's update rule applied to the GPU's own selection, every
cached row must equal its pool row, and the outputs must equal the uncached
offload path's bit for bit (and the oracle's attention within 2e-3)."""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth as S
from qsa_synth.device import DeviceInputs

from qsa_testlib import check_attention, check_selection, oracle_attention_on, oracle_unit

pytestmark = pytest.mark.gpu

qsa = pytest.importorskip("kv_cache_selection_amd")
G = S.GEOM


def _drifted(base_bits, rng, delta):
    x = S.bf16_bits_to_f32(base_bits) + np.float32(delta) * rng.standard_normal(base_bits.shape).astype(np.float32)
    return S.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("n_side", [0, 2])
def test_hot_cache_steps(gpu, n_side):
    wl = S.Workload("hot-test", 2, (20000, 13001), 2, 256, tail_tokens=0, planted=8, seed=7)
    di = DeviceInputs(wl, gpu, kv_host=True)
    hi = di.hi
    B, NL, H, K = di.batch, di.n_layers, 300, wl.budget // 4
    cfg = qsa.make_config(wl.budget, wl.sink_blocks, wl.tail_tokens, G.sm_scale)
    bt = qsa.make_batch(B, di.max_ctx, di.ctx, di.row0, di.pt, di.pt_stride, di.n_slots, di.n_rows)
    caches, miss = [], []
    for l in range(NL):
        rows = torch.zeros((B, H, G.row_elems), dtype=torch.int16, device=gpu)
        map_ = torch.zeros((B, di.pt_stride), dtype=torch.int32, device=gpu)
        owner = torch.zeros((B, H), dtype=torch.int32, device=gpu)
        nm = torch.zeros(B, dtype=torch.int32, device=gpu)
        hc = qsa.make_hot_cache(rows, map_, owner, H, nm)
        qsa.qsa_hot_reset(bt, hc)
        caches.append(hc)
        miss.append(nm)
    loc = qsa.QSA_KV_HOST_PINNED
    nws = qsa.qsa_workspace_size(cfg, B, di.max_ctx, NL, loc)
    ws = torch.empty(nws, dtype=torch.uint8, device=gpu)
    ref_map = [np.full((B, di.pt_stride), -1, np.int64) for _ in range(NL)]
    ref_own = [np.full((B, H), -1, np.int64) for _ in range(NL)]
    rng = np.random.default_rng(71)
    side = [torch.cuda.Stream() for _ in range(n_side)]
    ev = qsa.StepEvents(NL, n_side) if n_side else None
    base_q_idx = hi.q_idx.copy()
    n_fetched = []
    for step in range(4):
        # this step's queries: the indexer queries drift a little, the attention queries are fresh
        q_idx = np.stack([_drifted(base_q_idx[l], rng, 0.35) for l in range(NL)])
        q = np.stack([S.f32_to_bf16_bits(rng.standard_normal((B, G.n_q_heads, G.head_dim)).astype(np.float32))
                      for _ in range(NL)])
        d_qi = torch.from_numpy(q_idx.view(np.int16)).to(gpu)
        d_q = torch.from_numpy(q.view(np.int16)).to(gpu)
        sel = torch.full((NL, B, K), -1, dtype=torch.int32, device=gpu)
        ns = torch.zeros((NL, B), dtype=torch.int32, device=gpu)
        out_hot = torch.full((NL, B, G.n_q_heads, G.head_dim), float("nan"), device=gpu)
        out_plain = torch.full_like(out_hot, float("nan"))
        mk = lambda out, hot: [qsa.make_layer(di.keys[l], di.scales[l], d_qi[l], di.w_idx[l], d_q[l], di.pool[l],
                                              out[l], None, sel[l], ns[l], hot=hot[l] if hot else None)
                               for l in range(NL)]
        qsa.qsa_decode_step(cfg, bt, mk(out_hot, caches), loc, ws, nws, torch.cuda.current_stream(), side, events=ev)
        torch.cuda.synchronize()
        sel_h, ns_h = sel.cpu().numpy().copy(), ns.cpu().numpy().copy()
        qsa.qsa_decode_step(cfg, bt, mk(out_plain, None), loc, ws, nws, torch.cuda.current_stream(), side,
                            events=ev)
        torch.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), sel_h)
        assert np.array_equal(out_hot.cpu().numpy(), out_plain.cpu().numpy())      # the cache is transparent
        step_fetches = 0
        for l in range(NL):
            gmap = caches[l]._keep[1].cpu().numpy()
            gown = caches[l]._keep[2].cpu().numpy()
            grows = caches[l]._keep[0].cpu().numpy().view(np.uint16)
            gmiss = miss[l].cpu().numpy()
            for b in range(B):
                L = int(hi.lay.ctx[b])
                # the selection against the oracle (same drifted queries)
                hi.q_idx[l, b] = q_idx[l, b]
                u = oracle_unit(hi, l, b)
                got = sel_h[l, b, :ns_h[l, b]]
                check_selection(got, u)
                toks = oracle.tokens_of_blocks(L, got)
                f = oracle.hot_cache_update(ref_map[l][b], ref_own[l][b], toks, b, H)
                assert gmiss[b] == len(f), (step, l, b)
                step_fetches += len(f)
                assert np.array_equal(gmap[b], ref_map[l][b]), (step, l, b)
                assert np.array_equal(gown[b], ref_own[l][b]), (step, l, b)
                owned = np.nonzero(gown[b] >= 0)[0]
                host_rows = S.kv_rows(wl.seed, l, hi.lay.pt[b, gown[b, owned]])
                assert np.array_equal(grows[b, owned], host_rows), (step, l, b)
                hi.q[l, b] = q[l, b]
                want = oracle_attention_on(hi, l, b, toks)
                check_attention(out_hot[l, b].cpu().numpy(), want, "hot l%d b%d" % (l, b))
        hi.q_idx[:] = base_q_idx
        n_fetched.append(step_fetches)
    # the first step fetches every selected row; later steps reuse the cache
    assert n_fetched[0] == NL * B * wl.budget
    assert all(n < n_fetched[0] for n in n_fetched[1:]), n_fetched


def test_hot_cache_rejects_bad_configurations(gpu):
    wl = S.WORKLOADS["tiny-4k"]
    di = DeviceInputs(wl, gpu)
    cfg = qsa.make_config(wl.budget)
    bt = qsa.make_batch(1, di.max_ctx, di.ctx, di.row0, di.pt, di.pt_stride, di.n_slots, di.n_rows)
    rows = torch.zeros((1, 512, G.row_elems), dtype=torch.int16, device=gpu)
    m = torch.zeros((1, di.pt_stride), dtype=torch.int32, device=gpu)
    o = torch.zeros((1, 512), dtype=torch.int32, device=gpu)
    out = torch.zeros((1, 16, 256), device=gpu)
    nws = qsa.qsa_workspace_size(cfg, 1, di.max_ctx, 1, qsa.QSA_KV_HOST_PINNED)
    ws = torch.empty(nws, dtype=torch.uint8, device=gpu)
    for hc, loc in [(qsa.make_hot_cache(rows, m, o, 512), qsa.QSA_KV_DEVICE),        # needs a host pool
                    (qsa.make_hot_cache(rows, m, o, 100), qsa.QSA_KV_HOST_PINNED)]:  # fewer rows than the budget
        lay = qsa.make_layer(di.keys[0], di.scales[0], di.q_idx[0], di.w_idx[0], di.q[0], di.pool[0], out, hot=hc)
        with pytest.raises(qsa.QsaError) as ei:
            qsa.qsa_decode_step(cfg, bt, [lay], loc, ws, nws)
        assert ei.value.status == qsa.QSA_ERR_INVALID_ARGUMENT
