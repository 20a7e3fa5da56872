"""Oracle parity at the workloads' full sizes, in the launch configuration the
benchmark times.

  - batch8-256k (8 x 262,144 tokens, 12 layers, sink 1): every sequence of
    layer 0 and two sequences through all 12 layers against the oracle;
  - offload-1m (1 x 1,048,576 tokens, 12 layers, KV in pinned host memory):
    the bench's schedule and the one-stream schedule give the same bits, and
    four layers match the oracle;
  - the block selection alone at 1,048,576 tokens (262,144 blocks, one
    output bitmap segment), just past it and at the 2,097,152-token limit
    (two segments), with random, tied and constant scores, sinks and tails.

The oracle runs on several host threads: its C code releases the GIL, and
each (layer, sequence) unit is independent.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import qsa_synth as S
from qsa_synth.device import DeviceInputs

from qsa_testlib import check_attention, check_selection, oracle_attention_on, oracle_unit

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

qsa = pytest.importorskip("kv_cache_selection_amd")
G = S.GEOM


def _step(di, n_side, loc):
    wl = di.wl
    cfg = qsa.make_config(wl.budget, wl.sink_blocks, wl.tail_tokens, G.sm_scale)
    K = wl.budget // 4
    L = di.n_layers
    sel = torch.full((L, di.batch, K), -7, dtype=torch.int32, device="cuda")
    ns = torch.zeros((L, di.batch), dtype=torch.int32, device="cuda")
    di.out.fill_(float("nan"))
    layers = [qsa.make_layer(di.keys[l], di.scales[l], di.q_idx[l], di.w_idx[l], di.q[l], di.pool[l], di.out[l],
                             None, sel[l], ns[l]) for l in range(L)]
    nws = qsa.qsa_workspace_size(cfg, di.batch, di.max_ctx, L, loc)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    side = [torch.cuda.Stream() for _ in range(n_side)]
    bt = qsa.make_batch(di.batch, di.max_ctx, di.ctx, di.row0, di.pt, di.pt_stride, di.n_slots, di.n_rows)
    ev = qsa.StepEvents(L, n_side) if n_side else None
    qsa.qsa_decode_step(cfg, bt, layers, loc, ws, nws, torch.cuda.current_stream(), side, events=ev)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), ns.cpu().numpy(), di.out.cpu().numpy()


def _check_units_threaded(di, sel, ns, out, units, threads=8):
    def one(unit):
        l, b = unit
        u = oracle_unit(di.hi, l, b)
        gsel = sel[l, b, :ns[l, b]]
        excused = check_selection(gsel, u)
        toks = u.tokens if np.array_equal(gsel, u.sel) else oracle.tokens_of_blocks(u.L, gsel)
        ref = oracle_attention_on(di.hi, l, b, toks)
        check_attention(out[l, b], ref, "unit %s" % (unit,))
        return excused

    with ThreadPoolExecutor(max_workers=threads) as ex:
        return sum(ex.map(one, units))


def test_decode_step_batch8_256k_sampled(gpu):
    """The whole 8 x 262,144 x 12-layer workload in the benchmark's launch
    configuration (one side stream): every sequence of layer 0 and sequences
    2 and 5 through all 12 layers against the oracle (30 units); in every
    unit the sink block and the planted blocks are selected."""
    di = DeviceInputs(S.WORKLOADS["batch8-256k"], gpu)
    sel, ns, out = _step(di, 1, qsa.QSA_KV_DEVICE)
    assert np.all(ns == 512)
    units = sorted({(0, b) for b in range(8)} | {(l, b) for l in range(12) for b in (2, 5)})
    assert len(units) == 30
    _check_units_threaded(di, sel, ns, out, units)
    for l in range(12):
        for b in range(8):
            assert sel[l, b, 0] == 0                           # the sink block
            assert set(di.hi.lay.planted[(l, b)].tolist()) <= set(sel[l, b].tolist())
    del di
    torch.cuda.empty_cache()


def test_decode_step_offload_1m(gpu):
    """The 1 x 1,048,576-token workload with all 12 layers' KV in pinned host
    memory (25.8 GB), in the bench's schedule (three side streams) and on one
    stream: the same bits, and layers 0, 3, 7 and 11 match the oracle."""
    di = DeviceInputs(S.WORKLOADS["offload-1m"], gpu)
    assert di.kv_host
    sel, ns, out = _step(di, 3, qsa.QSA_KV_HOST_PINNED)
    sel1, ns1, out1 = _step(di, 0, qsa.QSA_KV_HOST_PINNED)
    assert np.array_equal(sel, sel1) and np.array_equal(ns, ns1) and np.array_equal(out, out1)
    assert np.all(ns == 512)
    _check_units_threaded(di, sel, ns, out, [(0, 0), (3, 0), (7, 0), (11, 0)], threads=4)
    for l in range(12):
        assert set(di.hi.lay.planted[(l, 0)].tolist()) <= set(sel[l, 0].tolist())
    del di
    torch.cuda.empty_cache()


def _topk(budget, sink, tail, bs_rows, lens):
    cfg = qsa.make_config(budget, sink, tail)
    K = budget // 4
    B = len(lens)
    max_ctx = int(max(lens))
    ctx = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    bt = qsa.make_batch(B, max_ctx, ctx)
    nws = qsa.qsa_workspace_size(cfg, B, max_ctx, 1, qsa.QSA_KV_DEVICE)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ws.fill_(0xCD)                                   # arbitrary workspace content
    sel = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    ns = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    bs_d = torch.from_numpy(np.ascontiguousarray(bs_rows, np.float32)).cuda()
    qsa.qsa_topk_blocks(cfg, bt, bs_d, bs_rows.shape[1], sel, ns, nt, ws, nws)
    torch.cuda.synchronize()
    sel, ns, nt = sel.cpu().numpy(), ns.cpu().numpy(), nt.cpu().numpy()
    for b, L in enumerate(lens):
        n = (L + 3) // 4
        ref = oracle.select_blocks(bs_rows[b, :n], K, oracle.forced_mask(L, 4, sink, tail)).blocks
        assert ns[b] == len(ref), (b, L, ns[b], len(ref))
        assert np.array_equal(sel[b, :ns[b]], ref), (b, L)
        assert np.all(sel[b, ns[b]:] == -1)
        assert nt[b] == len(oracle.tokens_of_blocks(L, ref)), (b, L)


# 1,048,576 tokens fill exactly one 262,144-block segment of the selection
# kernel's output bitmap; one token more starts a second segment; 2,097,152
# tokens is the longest context the library accepts (two full segments).
LONG = [1048576, 1048577, 2097152]


@pytest.mark.parametrize("kind", ["random", "ties", "constant", "two-values", "clustered"])
def test_topk_exact_at_1m_and_2m_tokens(gpu, kind):
    rng = np.random.default_rng({"random": 31, "ties": 32, "constant": 33, "two-values": 34, "clustered": 35}[kind])
    lens = LONG + [4 * 512 + 3, 300001]
    n_max = (max(lens) + 3) // 4
    if kind == "random":
        bs = rng.standard_normal((len(lens), n_max)).astype(np.float32) * 10
        bs[:, ::11] = -0.0
    elif kind == "ties":
        bs = rng.integers(0, 50, size=(len(lens), n_max)).astype(np.float32)
    elif kind == "constant":
        bs = np.full((len(lens), n_max), 3.5, np.float32)
    elif kind == "clustered":                  # the answer crowded into a few chunks
        bs = rng.standard_normal((len(lens), n_max)).astype(np.float32)
        bs[:, 40000:41500] += 30.0
        bs[:, 270000:270400] += 25.0
    else:
        bs = np.full((len(lens), n_max), 3.5, np.float32)
        bs[:, 1::2] = np.nextafter(np.float32(3.5), np.float32(10))
    # the best blocks sit in the second segment for some sequences
    if kind == "random":
        bs[1, -5:] = 1e6
        bs[2, 262144 + 7] = 1e6
    for budget, sink, tail in ((2048, 1, 0), (2048, 0, 64), (8192, 2, 0), (4, 0, 0)):
        _topk(budget, sink, tail, bs, lens)
