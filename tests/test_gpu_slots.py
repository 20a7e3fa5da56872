"""Slot leases end to end on the GPU: tokens are placed by the library's slot
pool (tail ring + body slots), ring spills are moved with qsa_move_tokens,
tokens are appended with qsa_append_token, and the cache must hold every
token's row at the slot its page-table entry names, bit for bit. Generation
markers must flag exactly the entries of a closed lease, and a decode step
over the surviving request must match the oracle."""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth as S

from qsa_testlib import check_attention

pytestmark = pytest.mark.gpu

qsa = pytest.importorskip("kv_cache_selection_amd")
G = S.GEOM


def test_lease_lifecycle(gpu):
    rng = np.random.default_rng(61)
    B, NL, T, R, n_slots = 2, 2, 120, 16, 512
    pool = qsa.SlotPool(n_slots)
    model = oracle.SlotPoolModel(n_slots)
    leases = [pool.open(R) for _ in range(B)]
    mleases = [model.open(R) for _ in range(B)]
    stride = T
    row0 = np.array([0, T], np.int64)
    d_ctx = torch.zeros(B, dtype=torch.int32, device=gpu)
    d_row0 = torch.from_numpy(row0).to(gpu)
    d_pt = torch.full((B, stride), -1, dtype=torch.int32, device=gpu)
    d_gen = torch.zeros((B, stride), dtype=torch.int32, device=gpu)          # token generations (uint32 bits)
    keys = [torch.zeros((B * T, G.idx_dim), dtype=torch.uint8, device=gpu) for _ in range(NL)]
    scales = [torch.zeros(B * T, dtype=torch.int16, device=gpu) for _ in range(NL)]
    pools = [torch.zeros((n_slots, G.row_elems), dtype=torch.int16, device=gpu) for _ in range(NL)]
    cfg = qsa.make_config(256, 0, 16, G.sm_scale)
    bt = qsa.make_batch(B, stride, d_ctx, d_row0, d_pt, stride, n_slots, B * T)
    rows_ref = np.zeros((NL, B, T, G.row_elems), np.uint16)
    keys_ref = np.zeros((NL, B, T, G.idx_dim), np.float32)
    pt_ref = np.full((B, stride), -1, np.int64)
    for t in range(T):
        plans = [pool.next_token(lid) for lid in leases]
        mplans = [model.next_token(mid) for mid in mleases]
        for p, (slot, gen, spill) in zip(plans, mplans):
            assert (p.slot, p.generation) == (slot, gen) and p.token == t
            assert (p.spill_token, p.spill_to) == ((spill[0], spill[2]) if spill else (-1, -1))
        if any(p.spill_token >= 0 for p in plans):
            tok = torch.tensor([p.spill_token for p in plans], dtype=torch.int64, device=gpu)
            to = torch.tensor([p.spill_to for p in plans], dtype=torch.int32, device=gpu)
            tg = torch.tensor([p.spill_generation for p in plans], dtype=torch.int32, device=gpu)
            qsa.qsa_move_tokens(bt, pools, qsa.QSA_KV_DEVICE, tok, to, d_pt, tg, d_gen)
            for b, p in enumerate(plans):
                if p.spill_token >= 0:
                    pt_ref[b, p.spill_token] = p.spill_to
        nk = [rng.standard_normal((B, G.idx_dim)).astype(np.float32) for _ in range(NL)]
        nr = [S.f32_to_bf16_bits(rng.standard_normal((B, G.row_elems)).astype(np.float32)) for _ in range(NL)]
        for l in range(NL):
            rows_ref[l, :, t] = nr[l]
            keys_ref[l, :, t] = nk[l]
        layers = [qsa.make_append_layer(torch.from_numpy(nk[l]).to(gpu), torch.from_numpy(nr[l].view(np.int16)).to(gpu),
                                        keys[l], scales[l], pools[l]) for l in range(NL)]
        slots = torch.tensor([p.slot for p in plans], dtype=torch.int32, device=gpu)
        gens = torch.tensor([p.generation for p in plans], dtype=torch.int32, device=gpu)
        qsa.qsa_append_token(cfg, bt, layers, qsa.QSA_KV_DEVICE, slots, d_pt, d_ctx, new_gen=gens, tok_gen=d_gen)
        for b, p in enumerate(plans):
            pt_ref[b, t] = p.slot
    torch.cuda.synchronize()
    assert list(d_ctx.cpu().numpy()) == [T, T]
    pt = d_pt.cpu().numpy()
    assert np.array_equal(pt, pt_ref)
    # the last R tokens sit in the ring, the others in distinct body slots
    for b in range(B):
        ring = model.leases[mleases[b]]["ring"]
        assert [pt[b, t] for t in range(T - R, T)] == [ring[t % R] for t in range(T - R, T)]
    assert len(set(pt.reshape(-1).tolist())) == B * T
    for l in range(NL):
        got = pools[l].cpu().numpy().view(np.uint16)
        for b in range(B):
            assert np.array_equal(got[pt[b]], rows_ref[l, b]), (l, b)

    # generations: nothing is stale; after request 0 ends, all of its entries are
    slot_gen = torch.from_numpy(pool.generations().view(np.int32)).to(gpu)
    stale = torch.full((B,), -1, dtype=torch.int32, device=gpu)
    qsa.qsa_check_generations(bt, d_pt, d_gen, slot_gen, stale)
    torch.cuda.synchronize()
    assert list(stale.cpu().numpy()) == [0, 0]
    pool.close(leases[0])
    model.close(mleases[0])
    assert pool.free_slots() == model.free_slots() == n_slots - (T + 0)
    slot_gen = torch.from_numpy(pool.generations().view(np.int32)).to(gpu)
    qsa.qsa_check_generations(bt, d_pt, d_gen, slot_gen, stale)
    torch.cuda.synchronize()
    assert list(stale.cpu().numpy()) == [T, 0]

    # the surviving request decodes over its cache exactly as the oracle does
    b = 1
    q_idx = S.f32_to_bf16_bits(rng.standard_normal((B, G.idx_heads, G.idx_dim)).astype(np.float32))
    w = rng.uniform(0, 1, (B, G.idx_heads)).astype(np.float32)
    q = S.f32_to_bf16_bits(rng.standard_normal((B, G.n_q_heads, G.head_dim)).astype(np.float32))
    out = torch.zeros((B, G.n_q_heads, G.head_dim), device=gpu)
    sel = torch.full((B, 64), -1, dtype=torch.int32, device=gpu)
    ns = torch.zeros(B, dtype=torch.int32, device=gpu)
    lay = qsa.make_layer(keys[0], scales[0], torch.from_numpy(q_idx.view(np.int16)).to(gpu), torch.from_numpy(w).to(gpu),
                         torch.from_numpy(q.view(np.int16)).to(gpu), pools[0], out, None, sel, ns)
    nws = qsa.qsa_workspace_size(cfg, B, stride, 1)
    ws = torch.empty(nws, dtype=torch.uint8, device=gpu)
    qsa.qsa_decode_step(cfg, bt, [lay], qsa.QSA_KV_DEVICE, ws, nws, torch.cuda.current_stream())
    torch.cuda.synchronize()
    # the oracle's inputs come from the host: its own quantisation of the keys
    # and a pool holding each appended row at the slot the reference placed it
    kh = np.zeros((T, G.idx_dim), np.uint8)
    sh = np.zeros(T, np.uint16)
    for t in range(T):
        kh[t], sh[t] = oracle.quantise_key(keys_ref[0, b, t])
    host_pool = np.zeros((n_slots, G.row_elems), np.uint16)
    host_pool[pt_ref[b]] = rows_ref[0, b]
    ts = oracle.token_scores(kh, sh, q_idx[b], w[b])
    bs = oracle.block_scores(ts)
    ref = oracle.select_blocks(bs, 64, oracle.forced_mask(T, 4, 0, 16))
    got = sel[b, :int(ns[b])].cpu().numpy()
    assert len(got) == len(ref.blocks) == T // 4                    # the budget covers the whole request
    toks = oracle.tokens_of_blocks(T, got)
    want = oracle.attention(toks, pt_ref[b].astype(np.int32), host_pool, q[b], G.n_kv_heads, G.sm_scale)
    check_attention(out[b].cpu().numpy(), want, "slots")
    # and that is attention over the rows the request appended
    dense = oracle.attention(np.arange(T), None, rows_ref[0, b], q[b], G.n_kv_heads, G.sm_scale)
    assert np.abs(want - dense).max() <= 1e-6
