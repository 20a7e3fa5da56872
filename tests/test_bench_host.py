"""Host-side logic of bench.py, without a GPU: the counter summary and its
copy calibration, the traffic lookup guarded by the scoring kernel's source
hash, the count of tokens a selection covers, and the CPU baseline on a small
workload."""
import csv

import numpy as np

import bench
import oracle
import qsa_synth as S

SCORE_GROUP = "void qsa::(anonymous namespace)::index_score_kernel<false, true, 16>(qsa::ScoreLayersT<16>, int const*)"
SCORE_LAYER = "void qsa::(anonymous namespace)::index_score_kernel<false, true, 1>(qsa::ScoreLayersT<1>, int const*)"
COPY = "__amd_rocclr_copyBuffer"


def _counters(path, rows):
    """A rocprofv3 counter_collection.csv: one row per dispatch and counter."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, counter, value) in enumerate(rows):
            w.writerow([i, name, counter, value])


def _summary(tmp_path):
    f, w, cf, cw = (str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    _counters(f, [(SCORE_GROUP, "FETCH_SIZE", 800000.0), (SCORE_GROUP, "FETCH_SIZE", 820000.0),
                  (SCORE_LAYER, "FETCH_SIZE", 67000.0)])
    _counters(w, [(SCORE_GROUP, "WRITE_SIZE", 25000.0), (SCORE_GROUP, "WRITE_SIZE", 25000.0),
                  (SCORE_LAYER, "WRITE_SIZE", 2000.0)])
    # The calibration copy moves COPY_BYTES each way: here FETCH_SIZE counts
    # 2-byte units of a KiB and WRITE_SIZE bytes of a KiB; a small dispatch of
    # the same run is not the copy.
    _counters(cf, [(COPY, "FETCH_SIZE", bench.COPY_BYTES / 2 / 1024), (COPY, "FETCH_SIZE", 3.0)])
    _counters(cw, [(COPY, "WRITE_SIZE", bench.COPY_BYTES / 1024), (COPY, "WRITE_SIZE", 1.0)])
    return bench.pmc_summary([f, w, cf, cw], "unit-test")


def _fields(text):
    out = {}
    for line in text.splitlines():
        if line and not line.startswith("#") and not line[0].isspace() and ":" in line:
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def test_pmc_summary_calibrates_and_averages(tmp_path):
    kv = _fields(_summary(tmp_path))
    assert float(kv["fetch_factor"]) == 2.0
    assert float(kv["write_factor"]) == 1.0
    # mean of the dispatches, KiB -> bytes through each counter's factor
    assert int(kv["traffic_bytes_per_group_launch"]) == 810000 * 1024 * 2 + 25000 * 1024
    assert int(kv["traffic_bytes_per_layer_launch"]) == 67000 * 1024 * 2 + 2000 * 1024
    assert kv["source_sha256"] == bench.score_source_hash()


def test_read_traffic_only_for_the_current_scoring_source(tmp_path, monkeypatch):
    text = _summary(tmp_path)
    path = tmp_path / "summary.txt"
    path.write_text(text)
    monkeypatch.setattr(bench, "pmc_file", lambda workload: str(path))
    assert bench.read_traffic("unit-test", True) == 810000 * 1024 * 2 + 25000 * 1024
    assert bench.read_traffic("unit-test", False) == 67000 * 1024 * 2 + 2000 * 1024
    # counters taken on another version of the kernel are not reported
    path.write_text(text.replace(bench.score_source_hash(), "0" * 64))
    assert bench.read_traffic("unit-test", True) is None
    monkeypatch.setattr(bench, "pmc_file", lambda workload: str(tmp_path / "missing.txt"))
    assert bench.read_traffic("unit-test", True) is None


def test_tokens_selected_matches_the_oracle_token_sets():
    ctx = np.array([4097, 10, 0, 2048])
    sels = [np.array([0, 5, 1024]),           # last block partial: 1 token
            np.array([0, 1, 2]),              # 10 tokens, last block 2 tokens
            np.array([], np.int64),           # empty sequence
            np.arange(512)]                   # every block, all whole
    K = 512
    sel = np.full((1, len(ctx), K), -1, np.int32)
    ns = np.zeros((1, len(ctx)), np.int32)
    for b, s in enumerate(sels):
        sel[0, b, :len(s)] = s
        ns[0, b] = len(s)
    got = bench.tokens_selected(sel, ns, ctx)
    want = [len(oracle.tokens_of_blocks(int(ctx[b]), sels[b])) for b in range(len(ctx))]
    assert got[0].tolist() == want == [9, 10, 0, 2048]


def test_cpu_baseline_reports_all_cores_and_one_core():
    wl = S.WORKLOADS["tiny-4k"]
    r = bench.cpu_baseline(wl, S.host_inputs(wl), 0.5)
    assert r["kind"] == "oracle" and r["unit"] == "layer-steps/s"
    assert r["cores"] >= 1 and r["value"] > 0
    one = r.get("single_core", r)
    assert one["cores"] == 1 and one["value"] > 0
