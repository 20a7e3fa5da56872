"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol the header declares, and rejects bad arguments before enqueuing any
work. Nothing here launches a kernel: every call returns during host-side
validation."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libqsa.h")

qsa = pytest.importorskip("kv_cache_selection_amd")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:qsa_status_t|size_t|void|int64_t|const char \*)\s*\*?\s*(qsa_\w+)\s*\(",
                                 txt, re.M)))


def test_header_declares_the_calls_and_helpers():
    names = _declared()
    for f in ("qsa_index_score", "qsa_topk_blocks", "qsa_gather_kv", "qsa_sparse_decode", "qsa_decode_step",
              "qsa_workspace_size", "qsa_layer_bytes", "qsa_status_string"):
        assert f in names
    assert set(names) == set(qsa.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(qsa.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    assert qsa.status_string(qsa.QSA_OK) == "ok"
    assert "workspace" in qsa.status_string(qsa.QSA_ERR_WORKSPACE_TOO_SMALL)
    assert qsa.status_string(99) == "unknown status"


def test_layer_bytes_match_the_pages():
    """66 B per index row and 2048 B per KV row; 2048 rows x 12 layers = 48 MiB."""
    cfg = qsa.make_config(2048)
    idx, kv = qsa.qsa_layer_bytes(cfg, 262144, 2048)
    assert idx == 66 * 262144 and kv == 2048 * 2048
    assert 12 * kv == 48 * 2**20


def test_workspace_size_grows_with_layers_and_offload():
    cfg = qsa.make_config(2048, sink_blocks=1)
    one = qsa.qsa_workspace_size(cfg, 8, 262144, 1)
    twelve = qsa.qsa_workspace_size(cfg, 8, 262144, 12)
    off = qsa.qsa_workspace_size(cfg, 1, 1 << 20, 12, qsa.QSA_KV_HOST_PINNED)
    assert one > 0 and twelve > 11 * one // 2 and off > 2 * 2048 * 2048
    assert qsa.qsa_workspace_size(cfg, 0, 100, 1) == 0
    assert qsa.qsa_workspace_size(cfg, 1, (1 << 21) + 1, 1) == 0
    assert qsa.qsa_workspace_size(qsa.make_config(6), 1, 100, 1) == 0     # budget not a multiple of 4


FAKE = 1 << 20      # a 256-byte aligned non-null address; never dereferenced on the host


def _batch(**kw):
    args = dict(batch=1, max_ctx=100, ctx_len=FAKE, idx_row0=FAKE, page_table=FAKE, pt_stride=100, n_slots=100,
                n_idx_rows=100)
    args.update(kw)
    return qsa.make_batch(**args)


@pytest.mark.parametrize("cfg_kw,status", [
    (dict(head_dim=128), qsa.QSA_ERR_UNSUPPORTED),
    (dict(n_q_heads=32), qsa.QSA_ERR_UNSUPPORTED),
    (dict(idx_dim=128), qsa.QSA_ERR_UNSUPPORTED),
    (dict(block_tokens=8), qsa.QSA_ERR_UNSUPPORTED),
    (dict(budget_tokens=2050), qsa.QSA_ERR_INVALID_ARGUMENT),
    (dict(budget_tokens=0), qsa.QSA_ERR_INVALID_ARGUMENT),
    (dict(budget_tokens=16384), qsa.QSA_ERR_INVALID_ARGUMENT),
    (dict(sink_blocks=-1), qsa.QSA_ERR_INVALID_ARGUMENT),
    (dict(budget_tokens=64, tail_tokens=64), qsa.QSA_ERR_INVALID_ARGUMENT),   # 17 forced blocks > 16
    (dict(budget_tokens=64, sink_blocks=17), qsa.QSA_ERR_INVALID_ARGUMENT),
])
def test_bad_config_rejected(cfg_kw, status):
    kw = dict(budget_tokens=2048)
    kw.update(cfg_kw)
    cfg = qsa.make_config(**kw)
    with pytest.raises(qsa.QsaError) as ei:
        qsa.qsa_index_score(cfg, _batch(), FAKE, FAKE, FAKE, FAKE, None, FAKE, 25)
    assert ei.value.status == status


def test_bad_arguments_rejected_before_launch():
    cfg = qsa.make_config(256)
    E = qsa.QSA_ERR_INVALID_ARGUMENT
    cases = [
        lambda: qsa.qsa_index_score(cfg, _batch(), None, FAKE, FAKE, FAKE, None, FAKE, 25),
        lambda: qsa.qsa_index_score(cfg, _batch(), FAKE + 4, FAKE, FAKE, FAKE, None, FAKE, 25),  # misaligned keys
        lambda: qsa.qsa_index_score(cfg, _batch(), FAKE, FAKE, FAKE, FAKE, None, FAKE, 24),      # bs_stride short
        lambda: qsa.qsa_index_score(cfg, _batch(batch=0), FAKE, FAKE, FAKE, FAKE, None, FAKE, 25),
        lambda: qsa.qsa_index_score(cfg, _batch(max_ctx=(1 << 21) + 1), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20),
        lambda: qsa.qsa_gather_kv(cfg, _batch(pt_stride=99), FAKE, FAKE, FAKE, 0, FAKE, FAKE),
        lambda: qsa.qsa_gather_kv(cfg, _batch(), FAKE, FAKE, FAKE + 8, 0, FAKE, FAKE),           # misaligned pool
        lambda: qsa.qsa_gather_kv(cfg, _batch(), FAKE, FAKE, FAKE, 7, FAKE, FAKE),               # bad location
        lambda: qsa.qsa_sparse_decode(cfg, 1, FAKE, FAKE, FAKE, FAKE, FAKE + 64, 1 << 30),       # misaligned ws
        lambda: qsa.qsa_sparse_decode(cfg, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30),
        lambda: qsa.qsa_decode_step(cfg, _batch(), [], 0, FAKE, 1 << 30),
        lambda: qsa.qsa_decode_step(cfg, _batch(), [qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)],
                                    0, FAKE, 1 << 30),                                           # no output
        lambda: qsa.qsa_decode_step(cfg, _batch(), [qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)],
                                    0, FAKE, 1 << 30, 4096, [4096]),                             # side == compute
        lambda: qsa.qsa_decode_step(cfg, _batch(), [qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)],
                                    0, FAKE, 1 << 30, 4096, [8192, 8192]),                       # repeated side
        lambda: qsa.qsa_decode_step(cfg, _batch(), [qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)],
                                    0, FAKE, 1 << 30, 4096, list(range(8192, 8192 + 9))),        # too many
        lambda: qsa.qsa_decode_step(cfg, _batch(), [qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)] * 65,
                                    0, FAKE, 1 << 30),                                           # > 64 layers
        # the kernels read 16-byte pieces of the queries and 4-byte words of the weights
        lambda: qsa.qsa_index_score(cfg, _batch(), FAKE, FAKE, FAKE + 8, FAKE, None, FAKE, 25),  # q_idx at 8
        lambda: qsa.qsa_index_score(cfg, _batch(), FAKE, FAKE + 1, FAKE, FAKE, None, FAKE, 25),  # odd scales
        lambda: qsa.qsa_index_score(cfg, _batch(), FAKE, FAKE, FAKE, FAKE + 2, None, FAKE, 25),  # w_idx at 2
        lambda: qsa.qsa_index_score_multi(cfg, _batch(), 4, FAKE, FAKE, FAKE, FAKE + 4, FAKE, FAKE, 25),
        lambda: qsa.qsa_index_score_multi(cfg, _batch(), 4, FAKE, FAKE, FAKE + 8, FAKE, FAKE, FAKE, 25),
        lambda: qsa.qsa_sparse_decode(cfg, 1, FAKE + 8, FAKE, FAKE, FAKE, FAKE, 1 << 30),       # q at 8
        lambda: qsa.qsa_decode_step(cfg, _batch(), [qsa.make_layer(FAKE, FAKE, FAKE + 8, FAKE, FAKE, FAKE, FAKE)],
                                    0, FAKE, 1 << 30),                                           # q_idx at 8
        lambda: qsa.qsa_decode_step(cfg, _batch(), [qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, FAKE)],
                                    0, FAKE, 1 << 30),                                           # q at 8
        lambda: qsa.qsa_read_flags(FAKE, None),
        lambda: qsa.qsa_read_flags(FAKE + 4, FAKE),                                              # ws not 256-aligned
        lambda: qsa.qsa_read_flags(FAKE, FAKE + 2),
    ]
    for i, c in enumerate(cases):
        with pytest.raises(qsa.QsaError) as ei:
            c()
        assert ei.value.status == E, i


def test_step_events_required_and_validated():
    """The schedules that order several streams (side streams with pools in
    pinned host memory, with or without a hot cache, or more than 16 layers
    on HBM pools with side streams) need a caller-made event set; the library
    creates no HIP object inside a call."""
    cfg = qsa.make_config(256)
    hc = qsa.make_hot_cache(FAKE, FAKE, FAKE, 256)
    lay_hot = qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, hot=hc)
    lay = qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for layers, loc in [([lay_hot] * 2, qsa.QSA_KV_HOST_PINNED), ([lay] * 2, qsa.QSA_KV_HOST_PINNED),
                        ([lay] * 17, qsa.QSA_KV_DEVICE)]:
        with pytest.raises(qsa.QsaError) as ei:
            qsa.qsa_decode_step(cfg, _batch(), layers, loc, FAKE, 1 << 34, 4096, [8192])
        assert ei.value.status == qsa.QSA_ERR_INVALID_ARGUMENT
    for bad in ((0, 1), (4, -1), (4, qsa.QSA_MAX_SIDE_STREAMS + 1)):
        with pytest.raises(qsa.QsaError) as ei:
            qsa.StepEvents(*bad)
        assert ei.value.status == qsa.QSA_ERR_INVALID_ARGUMENT
    assert qsa.lib.qsa_step_events_create(4, 1, None) == qsa.QSA_ERR_INVALID_ARGUMENT
    qsa.lib.qsa_step_events_destroy(None)          # a no-op


def test_workspace_too_small_rejected():
    cfg = qsa.make_config(256)
    need = qsa.qsa_workspace_size(cfg, 1, 100, 1)
    with pytest.raises(qsa.QsaError) as ei:
        qsa.qsa_topk_blocks(cfg, _batch(), FAKE, 25, FAKE, FAKE, None, FAKE, need - 1)
    assert ei.value.status == qsa.QSA_ERR_WORKSPACE_TOO_SMALL
    lay = qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    need = qsa.qsa_workspace_size(cfg, 1, 100, 2)
    with pytest.raises(qsa.QsaError) as ei:
        qsa.qsa_decode_step(cfg, _batch(), [lay, lay], 0, FAKE, need - 256)
    assert ei.value.status == qsa.QSA_ERR_WORKSPACE_TOO_SMALL


def test_structs_keep_their_tensors_alive():
    """The structs hold raw addresses; the binding keeps the tensors behind
    them referenced so their memory cannot be freed and reused before a call
    reads it (a freed row-offset tensor once sent the scoring kernel to
    addresses outside the index buffer)."""
    import gc
    import weakref
    torch = pytest.importorskip("torch")
    t = torch.zeros(4, dtype=torch.int32)
    r = weakref.ref(t)
    b = qsa.make_batch(1, 4, t, torch.zeros(1, dtype=torch.int64), n_idx_rows=4)
    del t
    gc.collect()
    assert r() is not None and b._keep[0] is r()
    k = torch.zeros(16, dtype=torch.uint8)
    rk = weakref.ref(k)
    lay = qsa.make_layer(k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    del k
    gc.collect()
    assert rk() is not None and lay.idx_keys == rk().data_ptr()
    with pytest.raises(ValueError):
        qsa.make_batch(1, 4, FAKE, FAKE)          # index rows without their count


def test_append_bad_arguments_rejected():
    cfg = qsa.make_config(256)
    E = qsa.QSA_ERR_INVALID_ARGUMENT
    good = qsa.make_append_layer(FAKE, FAKE, FAKE, FAKE, FAKE)
    cases = [
        lambda: qsa.qsa_append_token(cfg, _batch(), [], 0, FAKE, FAKE),                          # no layers
        lambda: qsa.qsa_append_token(cfg, _batch(), [good] * 65, 0, FAKE, FAKE),                 # too many
        lambda: qsa.qsa_append_token(cfg, _batch(), [good], 0, None, FAKE),                      # no slots
        lambda: qsa.qsa_append_token(cfg, _batch(), [good], 0, FAKE, None),                      # no table
        lambda: qsa.qsa_append_token(cfg, _batch(), [good], 5, FAKE, FAKE),                      # bad location
        lambda: qsa.qsa_append_token(cfg, _batch(), [qsa.make_append_layer(FAKE, FAKE + 8, FAKE, FAKE, FAKE)],
                                     0, FAKE, FAKE),                                             # misaligned row
        lambda: qsa.qsa_append_token(cfg, _batch(), [qsa.make_append_layer(None, FAKE, FAKE, FAKE, FAKE)],
                                     0, FAKE, FAKE),
        lambda: qsa.qsa_append_token(cfg, _batch(n_slots=0), [good], 0, FAKE, FAKE),
    ]
    for i, c in enumerate(cases):
        with pytest.raises(qsa.QsaError) as ei:
            c()
        assert ei.value.status == E, i
    with pytest.raises(qsa.QsaError) as ei:
        qsa.qsa_append_token(qsa.make_config(2048, head_dim=128), _batch(), [good], 0, FAKE, FAKE)
    assert ei.value.status == qsa.QSA_ERR_UNSUPPORTED


def test_hot_cache_bad_configurations_rejected():
    cfg = qsa.make_config(256)
    ok = qsa.make_hot_cache(FAKE, FAKE, FAKE, 256)
    small = qsa.make_hot_cache(FAKE, FAKE, FAKE, 255)
    huge = qsa.make_hot_cache(FAKE, FAKE, FAKE, 16385)
    lay = lambda hc: qsa.make_layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, hot=hc)
    E = qsa.QSA_ERR_INVALID_ARGUMENT
    for layers, loc in [([lay(ok)], qsa.QSA_KV_DEVICE), ([lay(small)], qsa.QSA_KV_HOST_PINNED),
                        ([lay(huge)], qsa.QSA_KV_HOST_PINNED), ([lay(ok), lay(None)], qsa.QSA_KV_HOST_PINNED)]:
        with pytest.raises(qsa.QsaError) as ei:
            qsa.qsa_decode_step(cfg, _batch(), layers, loc, FAKE, 1 << 30)
        assert ei.value.status == E
    with pytest.raises(qsa.QsaError) as ei:
        qsa.qsa_hot_reset(_batch(), huge)
    assert ei.value.status == E


def test_slot_pool_matches_the_reference_model():
    """The library's slot pool (host C++) gives the oracle model's plans, free
    counts and generations under random interleavings of opens, appends and
    closes, including exhaustion."""
    import numpy as np
    oracle = pytest.importorskip("oracle")
    rng = np.random.default_rng(52)
    pool = qsa.SlotPool(48)
    model = oracle.SlotPoolModel(48)
    ids = []                                      # (library id, model id)
    for _ in range(3000):
        r = rng.random()
        if r < 0.12 or not ids:
            ring = int(rng.integers(0, 6))
            try:
                mid = model.open(ring)
            except MemoryError:
                with pytest.raises(qsa.QsaError) as ei:
                    pool.open(ring)
                assert ei.value.status == qsa.QSA_ERR_OUT_OF_SLOTS
                continue
            ids.append((pool.open(ring), mid))
        elif r < 0.2:
            lid, mid = ids.pop(int(rng.integers(0, len(ids))))
            pool.close(lid)
            model.close(mid)
        else:
            lid, mid = ids[int(rng.integers(0, len(ids)))]
            try:
                slot, gen, spill = model.next_token(mid)
            except MemoryError:
                with pytest.raises(qsa.QsaError) as ei:
                    pool.next_token(lid)
                assert ei.value.status == qsa.QSA_ERR_OUT_OF_SLOTS
                continue
            p = pool.next_token(lid)
            assert (p.slot, p.generation) == (slot, gen)
            if spill is None:
                assert p.spill_token == -1 and p.spill_to == -1
            else:
                assert (p.spill_token, p.spill_from, p.spill_to, p.spill_generation) == spill
        assert pool.free_slots() == model.free_slots()
    for lid, mid in ids:
        pool.close(lid)
        model.close(mid)
    assert pool.free_slots() == 48
    assert list(pool.generations()) == model.gen
    with pytest.raises(qsa.QsaError):
        pool.close(12345)
