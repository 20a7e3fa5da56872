"""qsa_decode_step_static (the entry point that allocates nothing: its
workspace is the library's static device scratch) against qsa_decode_step
with a caller workspace, through the C ABI: bit-identical selections and
outputs on two calls in a row, the second with a smaller input, on one
stream and with a side stream; the flags word of the static scratch; and a
request larger than the scratch is refused before anything is enqueued."""
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


def _run(di, n_layers, static, n_side):
    wl = di.wl
    cfg = qsa.make_config(wl.budget, wl.sink_blocks, wl.tail_tokens, G.sm_scale)
    K = wl.budget // 4
    loc = qsa.QSA_KV_HOST_PINNED if di.kv_host else qsa.QSA_KV_DEVICE
    sel = torch.full((n_layers, di.batch, K), -7, dtype=torch.int32, device="cuda")
    ns = torch.full((n_layers, di.batch), -7, dtype=torch.int32, device="cuda")
    out = torch.full((n_layers, di.batch, G.n_q_heads, G.head_dim), float("nan"), device="cuda")
    layers = [qsa.make_layer(di.keys[l], di.scales[l], di.q_idx[l], di.w_idx[l], di.q[l], di.pool[l], out[l],
                             None, sel[l], ns[l]) for l in range(n_layers)]
    bt = qsa.make_batch(di.batch, di.max_ctx, di.ctx, di.row0, di.pt, di.pt_stride, di.n_slots, di.n_rows)
    side = [torch.cuda.Stream() for _ in range(n_side)]
    stream = torch.cuda.current_stream()
    if static:
        nws = qsa.qsa_workspace_size(cfg, di.batch, di.max_ctx, n_layers, loc)
        assert 0 < nws <= qsa.QSA_STATIC_SCRATCH_BYTES
        qsa.qsa_decode_step_static(cfg, bt, layers, loc, stream, side)
    else:
        nws = qsa.qsa_workspace_size(cfg, di.batch, di.max_ctx, n_layers, loc)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        qsa.qsa_decode_step(cfg, bt, layers, loc, ws, nws, stream, side)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), ns.cpu().numpy(), out.cpu().numpy()


def test_static_matches_workspace_entry_on_two_calls(gpu):
    big = DeviceInputs(S.WORKLOADS["batch8-short"], gpu, layers=3)
    small = DeviceInputs(S.WORKLOADS["tiny-4k"], gpu)
    for n_side in (0, 1):
        for di, n_layers in ((big, 3), (small, 1)):           # the second call is smaller
            want = _run(di, n_layers, False, n_side)
            got = _run(di, n_layers, True, n_side)
            for w, g in zip(want, got):
                assert np.array_equal(w, g), (di.wl.name, n_side)
            sel, ns, out = got
            for (l, b) in [(0, 0), (n_layers - 1, di.batch - 1)]:
                u = oracle_unit(di.hi, l, b)
                gsel = sel[l, b, :ns[l, b]]
                check_selection(gsel, u)
                toks = u.tokens if np.array_equal(gsel, u.sel) else oracle.tokens_of_blocks(u.L, gsel)
                check_attention(out[l, b], oracle_attention_on(di.hi, l, b, toks))
    flags = torch.full((1,), -1, dtype=torch.int32, device=gpu)
    qsa.qsa_read_flags(None, flags)
    torch.cuda.synchronize()
    assert int(flags[0]) == 0


def test_static_refuses_requests_beyond_the_scratch(gpu):
    wl = S.WORKLOADS["batch8-256k"]
    cfg = qsa.make_config(wl.budget, wl.sink_blocks, wl.tail_tokens, G.sm_scale)
    assert qsa.qsa_workspace_size(cfg, 8, 262144, 12) > qsa.QSA_STATIC_SCRATCH_BYTES
    d = torch.zeros(64, dtype=torch.int64, device=gpu)
    bt = qsa.make_batch(8, 262144, d, d, d, 262144, 1 << 20, 8 * 262144)
    lay = qsa.make_layer(d, d, d, d, d, d, d)
    with pytest.raises(qsa.QsaError) as ei:
        qsa.qsa_decode_step_static(cfg, bt, [lay] * 12, qsa.QSA_KV_DEVICE)
    assert ei.value.status == qsa.QSA_ERR_WORKSPACE_TOO_SMALL
