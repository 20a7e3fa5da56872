"""Parity of the append step (qsa_append_token, through the C ABI) with the
oracle's reference append: quantised index rows, scales, pool rows, page
table and lengths must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import qsa_synth as S

from qsa_testlib import check_attention

pytestmark = pytest.mark.gpu

qsa = pytest.importorskip("kv_cache_selection_amd")
G = S.GEOM


def _new_keys(rng, B, kinds):
    """New index keys with mixed magnitudes: normal, tiny (subnormal scales),
    huge, all zero, and elements on exact e4m3 midpoints after scaling."""
    keys = np.empty((B, G.idx_dim), np.float32)
    for b in range(B):
        k = kinds[b % len(kinds)]
        if k == "normal":
            keys[b] = rng.standard_normal(G.idx_dim) * rng.uniform(0.05, 5)
        elif k == "tiny":
            keys[b] = rng.standard_normal(G.idx_dim) * 1e-5
        elif k == "huge":
            keys[b] = rng.standard_normal(G.idx_dim) * 3e4
        elif k == "zero":
            keys[b] = 0.0
        elif k == "ties":
            vals = np.array([oracle.decode_e4m3(c) for c in range(1, 0x7E)])
            mids = (vals[:-1] + vals[1:]) / 2
            keys[b] = rng.choice(mids, G.idx_dim) * rng.choice([-1, 1], G.idx_dim)
            keys[b, 0] = 448.0                  # scale exactly 1.0: the midpoints stay midpoints
    return keys


class State:
    """A small cache: B sequences with room for `room` more tokens each."""

    def __init__(self, rng, ctx, room, n_layers, n_slots, pinned=False):
        self.B = len(ctx)
        self.ctx = np.array(ctx, np.int32)
        cap = self.ctx + room
        self.row0 = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
        self.n_rows = int(cap.sum())
        self.pt_stride = int(cap.max())
        self.n_slots = n_slots
        self.pt = rng.integers(0, n_slots, (self.B, self.pt_stride)).astype(np.int32)
        self.keys = [rng.integers(0, 256, (self.n_rows, G.idx_dim)).astype(np.uint8) for _ in range(n_layers)]
        self.scales = [rng.integers(0, 2 ** 15, self.n_rows).astype(np.uint16) for _ in range(n_layers)]
        self.pools = [rng.integers(0, 2 ** 16, (n_slots, G.row_elems)).astype(np.uint16) for _ in range(n_layers)]
        dev = "cuda"
        self.d_ctx = torch.from_numpy(self.ctx.copy()).to(dev)
        self.d_row0 = torch.from_numpy(self.row0).to(dev)
        self.d_pt = torch.from_numpy(self.pt.copy()).to(dev)
        self.d_keys = [torch.from_numpy(k.copy()).to(dev) for k in self.keys]
        self.d_scales = [torch.from_numpy(s.view(np.int16).copy()).to(dev) for s in self.scales]
        if pinned:
            self.d_pools = [torch.from_numpy(p.view(np.int16).copy()).pin_memory() for p in self.pools]
        else:
            self.d_pools = [torch.from_numpy(p.view(np.int16).copy()).to(dev) for p in self.pools]
        self.loc = qsa.QSA_KV_HOST_PINNED if pinned else qsa.QSA_KV_DEVICE

    def append(self, new_keys, new_rows, slots):
        """GPU append, then the oracle's on the host copies; compare."""
        cfg = qsa.make_config(256)
        bt = qsa.make_batch(self.B, self.pt_stride, self.d_ctx, self.d_row0, self.d_pt, self.pt_stride,
                            self.n_slots, self.n_rows)
        d_nk = [torch.from_numpy(k).cuda() for k in new_keys]
        d_nr = [torch.from_numpy(r.view(np.int16)).cuda() for r in new_rows]
        layers = [qsa.make_append_layer(d_nk[l], d_nr[l], self.d_keys[l], self.d_scales[l], self.d_pools[l])
                  for l in range(len(new_keys))]
        d_slot = torch.from_numpy(np.asarray(slots, np.int32)).cuda()
        qsa.qsa_append_token(cfg, bt, layers, self.loc, d_slot, self.d_pt, self.d_ctx)
        torch.cuda.synchronize()
        ok = np.array([0 <= s < self.n_slots and 0 <= c < self.pt_stride and self.row0[b] + c < self.n_rows
                       for b, (s, c) in enumerate(zip(slots, self.ctx))])
        want_ctx = self.ctx.copy()
        if ok.any():
            idx = np.nonzero(ok)[0]
            sub_pt = self.pt[idx]
            got_ctx = oracle.append_token(self.ctx[idx], self.row0[idx], sub_pt, np.asarray(slots)[idx],
                                          self.keys, self.scales, self.pools,
                                          [k[idx] for k in new_keys], [r[idx] for r in new_rows])
            self.pt[idx] = sub_pt
            want_ctx[idx] = got_ctx
        self.ctx = want_ctx
        assert np.array_equal(self.d_ctx.cpu().numpy(), self.ctx)
        assert np.array_equal(self.d_pt.cpu().numpy(), self.pt)
        for l in range(len(new_keys)):
            assert np.array_equal(self.d_keys[l].cpu().numpy(), self.keys[l]), l
            assert np.array_equal(self.d_scales[l].cpu().numpy().view(np.uint16), self.scales[l]), l
            assert np.array_equal(self.d_pools[l].cpu().numpy().view(np.uint16), self.pools[l]), l


@pytest.mark.parametrize("pinned", [False, True])
def test_append_bit_exact_three_rounds(gpu, pinned):
    rng = np.random.default_rng(31)
    st = State(rng, [5, 0, 17, 1], room=4, n_layers=3, n_slots=64, pinned=pinned)
    kinds = ["normal", "tiny", "huge", "zero", "ties"]
    for r in range(3):
        keys = [_new_keys(rng, st.B, kinds[r:] + kinds[:r]) for _ in range(3)]
        rows = [rng.integers(0, 2 ** 16, (st.B, G.row_elems)).astype(np.uint16) for _ in range(3)]
        slots = rng.choice(st.n_slots, st.B, replace=False)
        st.append(keys, rows, slots)


def test_append_rejected_sequences_are_untouched(gpu):
    """A slot outside the pool or a sequence without room leaves that
    sequence's cache and length as they were; the others are appended."""
    rng = np.random.default_rng(32)
    st = State(rng, [3, 6, 2], room=1, n_layers=2, n_slots=16)
    st.ctx[1] = st.pt_stride                              # no room left in the page table
    st.d_ctx.copy_(torch.from_numpy(st.ctx))
    keys = [_new_keys(rng, 3, ["normal"]) for _ in range(2)]
    rows = [rng.integers(0, 2 ** 16, (3, G.row_elems)).astype(np.uint16) for _ in range(2)]
    st.append(keys, rows, [4, 5, 16])                    # sequence 2: slot 16 is outside the pool
    assert list(st.ctx) == [4, st.pt_stride, 2]


def test_append_quantisation_many_keys(gpu):
    """1024 sequences append one token each: every key's codes and scale
    equal the oracle's nearest-value quantisation."""
    rng = np.random.default_rng(33)
    B = 1024
    st = State(rng, np.zeros(B, np.int32), room=1, n_layers=1, n_slots=B)
    keys = [(rng.standard_normal((B, G.idx_dim)) * np.exp(rng.uniform(-12, 10, (B, 1)))).astype(np.float32)]
    rows = [rng.integers(0, 2 ** 16, (B, G.row_elems)).astype(np.uint16)]
    st.append(keys, rows, rng.permutation(B))


def test_append_then_decode_attends_the_new_tokens(gpu):
    """The loop closes: tokens appended with a forced tail are selected by the
    next decode step, whose output matches the oracle's on the updated cache."""
    rng = np.random.default_rng(34)
    L0, room, n_slots = 600, 8, 1024
    st = State(rng, [L0], room=room, n_layers=1, n_slots=n_slots)
    # a coherent cache: quantised keys for the existing tokens, distinct slots
    codes, sig = S.quantise_rows(rng.standard_normal((L0, G.idx_dim)).astype(np.float32))
    st.keys[0][:L0] = codes
    st.scales[0][:L0] = sig
    perm = rng.permutation(n_slots).astype(np.int32)
    st.pt[0, :] = perm[:st.pt_stride]
    st.pools[0] = S.f32_to_bf16_bits(rng.standard_normal((n_slots, G.row_elems)).astype(np.float32))
    st.d_keys[0].copy_(torch.from_numpy(st.keys[0]))
    st.d_scales[0].copy_(torch.from_numpy(st.scales[0].view(np.int16)))
    st.d_pt.copy_(torch.from_numpy(st.pt))
    st.d_pools[0].copy_(torch.from_numpy(st.pools[0].view(np.int16)))
    for r in range(3):
        keys = [rng.standard_normal((1, G.idx_dim)).astype(np.float32)]
        rows = [S.f32_to_bf16_bits(rng.standard_normal((1, G.row_elems)).astype(np.float32))]
        st.append(keys, rows, [int(perm[L0 + r])])
    L = int(st.ctx[0])
    budget, tail = 256, 8
    cfg = qsa.make_config(budget, 0, tail, G.sm_scale)
    q_idx = S.f32_to_bf16_bits(rng.standard_normal((1, G.idx_heads, G.idx_dim)).astype(np.float32))
    w = rng.uniform(0, 1, (1, G.idx_heads)).astype(np.float32)
    q = S.f32_to_bf16_bits(rng.standard_normal((1, G.n_q_heads, G.head_dim)).astype(np.float32))
    out = torch.zeros((1, G.n_q_heads, G.head_dim), dtype=torch.float32, device="cuda")
    sel = torch.full((1, budget // 4), -1, dtype=torch.int32, device="cuda")
    ns = torch.zeros(1, dtype=torch.int32, device="cuda")
    lay = qsa.make_layer(st.d_keys[0], st.d_scales[0], torch.from_numpy(q_idx.view(np.int16)).cuda(),
                         torch.from_numpy(w).cuda(), torch.from_numpy(q.view(np.int16)).cuda(), st.d_pools[0], out,
                         None, sel, ns)
    bt = qsa.make_batch(1, st.pt_stride, st.d_ctx, st.d_row0, st.d_pt, st.pt_stride, n_slots, st.n_rows)
    nws = qsa.qsa_workspace_size(cfg, 1, st.pt_stride, 1)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    qsa.qsa_decode_step(cfg, bt, [lay], qsa.QSA_KV_DEVICE, ws, nws, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ts = oracle.token_scores(st.keys[0][:L], st.scales[0][:L], q_idx[0], w[0])
    bs = oracle.block_scores(ts)
    ref = oracle.select_blocks(bs, budget // 4, oracle.forced_mask(L, 4, 0, tail))
    got = sel[0, :int(ns[0])].cpu().numpy()
    assert len(got) == len(ref.blocks)
    assert set(range((L - tail) // 4, (L + 3) // 4)) <= set(got.tolist())       # the new tokens' blocks
    diff = np.setxor1d(got, ref.blocks)
    assert np.all(np.abs(bs[diff].astype(np.float64) - ref.kth_score) <= 1e-5 * abs(ref.kth_score)), diff
    toks = oracle.tokens_of_blocks(L, got)
    want = oracle.attention(toks, st.pt[0], st.pools[0], q[0], G.n_kv_heads, G.sm_scale)
    check_attention(out[0].cpu().numpy(), want, "append-then-decode")
