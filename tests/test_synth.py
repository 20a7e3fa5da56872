"""The seeded input generator: determinism, random access, encoders against
library conversions, and the structure the workloads call for."""
import numpy as np
import torch

import qsa_synth as S

MASK = 2**64 - 1


def _mix_py(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def test_splitmix_matches_python_integers():
    key = int(S.stream_key(7, S.T_KV, 3))
    assert key == _mix_py(((7 << 32) ^ (S.T_KV << 16) ^ 3) & MASK)
    c = np.array([0, 1, 2, 10**9, 2**40 + 5], np.uint64)
    got = S.outputs(key, c)
    for ci, g in zip(c.tolist(), got.tolist()):
        assert g == _mix_py((key + (ci + 1) * 0x9E3779B97F4A7C15) & MASK)


def test_splitmix_reference_sequence():
    """SplitMix64 seeded with 1234567 (state advanced by gamma before each output)
    gives the published sequence of the reference C implementation."""
    seq = S.outputs(np.uint64(1234567), np.arange(5, dtype=np.uint64)).tolist()
    assert seq == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_normals_exact_and_random_access():
    key = S.stream_key(1, S.T_Q, 0)
    idx = np.arange(1000, dtype=np.uint64)
    a = S.normals(key, idx)
    b = S.normals(key, idx[::-1])[::-1]
    assert np.array_equal(a, b)
    assert np.array_equal(S.normals(key, idx[500:510]), a[500:510])
    # integer numerators: value * 65536 is an integer
    assert np.all(a * 65536 == np.round(a * 65536))
    big = S.normals(key, np.arange(200000, dtype=np.uint64))
    assert abs(big.mean()) < 0.01 and abs(big.std() - 1) < 0.01


def test_bf16_encoder_matches_torch():
    x = (np.random.default_rng(0).standard_normal(100000) * 3).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(S.f32_to_bf16_bits(x), ref)


def test_e4m3_encoder_matches_torch_in_range():
    rng = np.random.default_rng(1)
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    sv = np.unique(vals[np.isfinite(vals)])
    mids = ((sv[1:].astype(np.float64) + sv[:-1]) / 2).astype(np.float32)
    x = np.concatenate([rng.standard_normal(50000) * 50, rng.standard_normal(50000) * 1e-2, sv, mids,
                        np.nextafter(mids, np.float32(1e9)), np.nextafter(mids, np.float32(-1e9))]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(S.f32_to_e4m3_codes(x), ref)
    assert S.f32_to_e4m3_codes(np.array([1e6, -500.0], np.float32)).tolist() == [0x7E, 0xFE]


def test_quantised_rows_reconstruct():
    x = S.normals(S.stream_key(0, S.T_IDXKEY, 0), np.arange(64 * 100, dtype=np.uint64)).reshape(100, 64)
    codes, sig = S.quantise_rows(x)
    dq = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy() * sig.view(np.float16)[:, None]
    assert np.all(np.abs(dq - x) <= np.abs(x) * 2**-3 + sig.view(np.float16)[:, None].astype(np.float64) * 2**-9)
    assert np.all(np.abs(torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()) <= 448)


def test_layouts_are_consistent():
    for name, wl in S.WORKLOADS.items():
        if wl.batch * max(wl.ctx or (wl.ragged[1],)) > 400000:
            continue
        lay = S.make_layout(wl)
        for b in range(wl.batch):
            L = int(lay.ctx[b])
            p = lay.pt[b, :L]
            assert p.min() >= 0 and p.max() < lay.n_slots
            for layer in range(wl.layers):
                pl = lay.planted[(layer, b)]
                assert len(pl) == min(wl.planted, len(pl)) and np.all(np.diff(pl) > 0)
                assert np.all(pl >= wl.sink_blocks)
                if wl.tail_tokens:
                    assert np.all(pl < (L - wl.tail_tokens) // 4)
        if wl.tail_tokens == 0:
            flat = np.concatenate([lay.pt[b, :lay.ctx[b]] for b in range(wl.batch)])
            assert len(np.unique(flat)) == len(flat)          # no slot shared
        else:
            for b in range(wl.batch):
                L = int(lay.ctx[b])
                tail = lay.pt[b, L - wl.tail_tokens:L]
                assert len(np.unique(tail)) == wl.tail_tokens  # one ring of distinct slots


def test_ragged_lengths_in_range():
    wl = S.WORKLOADS["batch8-short"]
    ctx = S.ctx_lengths(wl)
    assert len(ctx) == 8 and ctx.min() >= 3072 and ctx.max() <= 4608 and len(set(ctx.tolist())) > 1


def test_host_c_generator_matches_numpy():
    """The C version of the two large streams gives the numpy generator's bytes:
    index keys over a stretch that crosses planted blocks and a ragged end, KV
    rows at scattered slots, and the float32 -> float16 rounding of the scale
    against numpy's own conversion (normal, subnormal, overflow edges)."""
    from qsa_synth import host as SH
    SH.build(force=False)
    wl = S.WORKLOADS["batch8-256k"]
    hi = S.host_inputs(wl)
    for (l, b) in [(0, 0), (7, 3)]:
        pl = hi.lay.planted[(l, b)]
        for t0, t1 in [(0, 700), (int(pl[0]) * 4 - 37, int(pl[0]) * 4 + 541), (262144 - 301, 262144)]:
            c1, s1 = S.index_keys(wl.seed, l, b, t0, t1, pl, hi.u[l, b])
            c2, s2 = SH.index_keys(wl.seed, l, b, t0, t1, pl, hi.u[l, b])
            assert np.array_equal(c1, c2) and np.array_equal(s1, s2), (l, b, t0)
    slots = np.array([0, 1, 4095, 123457, 2**21 - 1])
    assert np.array_equal(S.kv_rows(wl.seed, 5, slots), SH.kv_rows(wl.seed, 5, slots))
    x = np.abs(np.random.default_rng(7).standard_normal(20000).astype(np.float32)) * np.float32(0.02)
    edges = np.float32([0.0, 1e-9, 2.0**-25, 3 * 2.0**-26, 2.0**-14, 2.0**-14 * 0.99, 65504, 65519.99, 65520, 7e4])
    x = np.concatenate([x, edges])
    got = np.array([SH.f32_to_f16_bits(float(v)) for v in x], np.uint16)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
