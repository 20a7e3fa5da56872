"""Seeded synthetic inputs for the QSA decode step.

This module produces inputs only: queries, indexer weights, quantised index
keys, KV rows, page tables, context lengths and planted relevant blocks. It
holds none of the method's arithmetic (no scoring, no selection, no
attention). Both the CPU oracle's callers and the GPU path draw their inputs
from here; large pools are filled on the GPU by ``fill.py``/``csrc/synth_fill.hip``,
which implement the same counter-based generator as the numpy code below, so
any row can be regenerated on the host bit for bit.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used in counter mode. A stream is named by
(seed, tensor id, layer); output c of the stream is mix64(key + (c+1)*gamma)
with key = mix64((seed << 32) ^ (tensor << 16) ^ layer).

Normals are Irwin-Hall sums of twelve 16-bit uniforms taken from three
consecutive outputs, centred exactly and scaled by 2^-16 -- an integer
computation converted to float32 once, hence identical on every device.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ------------------------------------------------------------ SplitMix64

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)

# tensor ids of the named streams
T_QIDX, T_W, T_Q, T_IDXKEY, T_PLANT_NOISE, T_KV, T_DRIFT, T_STEP_Q = 1, 2, 3, 4, 5, 6, 7, 8


def mix64(z):
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tensor: int, layer: int) -> np.uint64:
    return mix64(np.uint64(((int(seed) << 32) ^ (int(tensor) << 16) ^ int(layer)) & (2**64 - 1)))[()]


def outputs(key, counters):
    """Outputs of the stream `key` at the given counters (uint64 array)."""
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + (c + np.uint64(1)) * GAMMA)


def normals(key, idx, chunk: int = 1 << 20):
    """float32 N(0,1) draws (Irwin-Hall of 12) at normal indices `idx`.

    value = (sum of the twelve 16-bit chunks of outputs 3n, 3n+1, 3n+2 - 393210) / 65536,
    exact in float32 (|numerator| <= 393210 < 2^24)."""
    n = np.asarray(idx, dtype=np.uint64)
    shape = n.shape
    n = n.reshape(-1)
    out = np.empty(n.shape, np.float32)
    three = np.arange(3, dtype=np.uint64)[None, :]
    for a in range(0, n.size, chunk):
        c = n[a:a + chunk, None] * np.uint64(3) + three
        o = np.ascontiguousarray(outputs(key, c))            # [m][3] uint64
        acc = o.view(np.uint16).reshape(-1, 12).sum(axis=1, dtype=np.int64)
        out[a:a + chunk] = (acc - 393210).astype(np.float32) * np.float32(1.0 / 65536.0)
    return out.reshape(shape)


def uniforms(key, idx):
    """float32 U[0,1) draws: top 24 bits of output n, times 2^-24 (exact)."""
    o = outputs(key, idx)
    return ((o >> np.uint64(40)).astype(np.float32) * np.float32(2.0**-24)).astype(np.float32)


# --------------------------------------------------------------- encoders

def f32_to_bf16_bits(x):
    """Round float32 to bfloat16, nearest-even, as uint16 bits (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_e4m3_codes(x):
    """Round float32 to OCP E4M3FN codes, nearest-even, saturating to +-448."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    sign = ((u >> np.uint32(31)) << np.uint32(7)).astype(np.uint32)
    a = u & np.uint32(0x7FFFFFFF)
    af = a.view(np.float32)
    exp = (a >> np.uint32(23)).astype(np.int64) - 127
    # normal range (exponent >= -6): round the 23-bit mantissa to 3 bits
    r = ((a.astype(np.uint64) + np.uint64(0x7FFFF) + ((a >> np.uint32(20)) & np.uint32(1)).astype(np.uint64))
         >> np.uint64(20)).astype(np.int64) - (120 << 3)
    # subnormal range: value = m * 2^-9, m rounded to nearest even
    m = np.rint(af * np.float32(512.0)).astype(np.int64)
    code = np.where(exp >= -6, r, m)
    code = np.minimum(code, 0x7E)
    code = np.where(af >= np.float32(448.0), 0x7E, code)
    return (code.astype(np.uint32) | sign).astype(np.uint8)


def quantise_rows(x):
    """Per-row e4m3 quantisation of float32 rows [n][64]: sigma = fp16(amax/448),
    codes = e4m3(x / sigma). Returns (codes u8 [n][64], sigma bits u16 [n])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    sig16 = (amax / np.float32(448.0)).astype(np.float32).astype(np.float16)
    sig32 = sig16.astype(np.float32)
    safe = np.where(sig32 > 0, sig32, np.float32(1.0))
    codes = f32_to_e4m3_codes((x / safe[:, None]).astype(np.float32))
    codes[sig32 == 0] = 0
    return codes, sig16.view(np.uint16)


# ---------------------------------------------------------------- configs

@dataclass(frozen=True)
class Geometry:
    n_q_heads: int = 16
    n_kv_heads: int = 2
    head_dim: int = 256
    idx_heads: int = 4
    idx_dim: int = 64
    block_tokens: int = 4

    @property
    def row_elems(self) -> int:            # bf16 elements per KV row
        return 2 * self.n_kv_heads * self.head_dim

    @property
    def row_bytes(self) -> int:            # 2048
        return 2 * self.row_elems

    @property
    def index_row_bytes(self) -> int:      # 66
        return self.idx_dim + 2

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


GEOM = Geometry()


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    ctx: tuple            # per-sequence lengths, or None for ragged (drawn)
    layers: int
    budget: int
    sink_blocks: int = 0
    tail_tokens: int = 0
    planted: int = 8
    kv_host: bool = False
    ragged: tuple = None  # (lo, hi) inclusive for drawn lengths
    seed: int = 0
    hot_slots: int = 0    # rows of a hot cache per sequence and layer (0: none)
    drift: float = 0.0    # per-step noise on the indexer queries (see step_queries)
    step_variants: int = 1


WORKLOADS = {
    "tiny-4k": Workload("tiny-4k", 1, (4096,), 1, 256, planted=8, seed=0),
    "single-38k": Workload("single-38k", 1, (38912,), 12, 2048, planted=8, seed=1),
    "batch8-short": Workload("batch8-short", 8, None, 12, 2048, tail_tokens=64, planted=8,
                             ragged=(3072, 4608), seed=2),
    "batch8-256k": Workload("batch8-256k", 8, (262144,) * 8, 12, 2048, sink_blocks=1,
                            planted=32, seed=3),
    # the same batch at shorter contexts, for the fixed-budget context sweep
    "batch8-64k": Workload("batch8-64k", 8, (65536,) * 8, 12, 2048, sink_blocks=1, planted=32, seed=3),
    "batch8-16k": Workload("batch8-16k", 8, (16384,) * 8, 12, 2048, sink_blocks=1, planted=32, seed=3),
    "offload-1m": Workload("offload-1m", 1, (1048576,), 12, 2048, planted=8, kv_host=True, seed=4),
    "offload-1m-hot": Workload("offload-1m-hot", 1, (1048576,), 12, 2048, planted=8, kv_host=True, seed=4,
                               hot_slots=4096, drift=0.25, step_variants=8),
}


def ctx_lengths(wl: Workload) -> np.ndarray:
    if wl.ctx is not None:
        return np.array(wl.ctx, dtype=np.int64)
    lo, hi = wl.ragged
    rng = np.random.Generator(np.random.PCG64([wl.seed, 101]))
    return rng.integers(lo, hi + 1, size=wl.batch).astype(np.int64)


# ------------------------------------------------------------ small tensors

def q_idx_bits(seed: int, layer: int, batch: int, g: Geometry = GEOM):
    """Indexer queries, bf16 bits [B][idx_heads][idx_dim], N(0,1)."""
    n = np.arange(batch * g.idx_heads * g.idx_dim, dtype=np.uint64)
    v = normals(stream_key(seed, T_QIDX, layer), n)
    return f32_to_bf16_bits(v).reshape(batch, g.idx_heads, g.idx_dim)


def w_idx(seed: int, layer: int, batch: int, g: Geometry = GEOM):
    """Indexer head weights, float32 [B][idx_heads], U[0,1)."""
    n = np.arange(batch * g.idx_heads, dtype=np.uint64)
    return uniforms(stream_key(seed, T_W, layer), n).reshape(batch, g.idx_heads)


def q_bits(seed: int, layer: int, batch: int, g: Geometry = GEOM):
    """Attention queries, bf16 bits [B][n_q_heads][head_dim], N(0,1)."""
    n = np.arange(batch * g.n_q_heads * g.head_dim, dtype=np.uint64)
    v = normals(stream_key(seed, T_Q, layer), n)
    return f32_to_bf16_bits(v).reshape(batch, g.n_q_heads, g.head_dim)


def plant_direction(q_idx_b, w_b):
    """Planted key direction for one sequence-layer: u = sum_h w_h q_h (float64
    sum, rounded to float32). Planted tokens get keys u + 0.1 * noise."""
    q = bf16_bits_to_f32(q_idx_b).astype(np.float64)
    return (np.asarray(w_b, np.float64)[:, None] * q).sum(axis=0).astype(np.float32)


def planted_blocks(wl: Workload, layer: int, b: int, L: int, g: Geometry = GEOM):
    """Sorted distinct block indices that get planted keys; never a forced block."""
    n_blk = (L + g.block_tokens - 1) // g.block_tokens
    lo = wl.sink_blocks
    hi = n_blk
    if wl.tail_tokens > 0:
        hi = max(0, L - wl.tail_tokens) // g.block_tokens
    hi = min(hi, L // g.block_tokens)          # whole blocks only
    avail = max(hi - lo, 0)
    k = min(wl.planted, avail)
    rng = np.random.Generator(np.random.PCG64([wl.seed, 202, layer, b]))
    pick = rng.choice(avail, size=k, replace=False) + lo if k > 0 else np.zeros(0, np.int64)
    return np.sort(pick).astype(np.int32)


# ------------------------------------------------------------ index keys

def index_key_values(seed: int, layer: int, b: int, t0: int, t1: int, planted, u, g: Geometry = GEOM):
    """float32 index keys (before quantisation) of tokens [t0, t1) of sequence b."""
    t = np.arange(t0, t1, dtype=np.uint64)
    base = ((np.uint64(b) << np.uint64(28)) + t) * np.uint64(g.idx_dim)
    n = base[:, None] + np.arange(g.idx_dim, dtype=np.uint64)[None, :]
    x = normals(stream_key(seed, T_IDXKEY, layer), n)
    if len(planted):
        blk = (np.arange(t0, t1) // g.block_tokens)
        hit = np.isin(blk, np.asarray(planted))
        if hit.any():
            noise = normals(stream_key(seed, T_PLANT_NOISE, layer), n[hit])
            x[hit] = (np.asarray(u, np.float32)[None, :] + np.float32(0.1) * noise).astype(np.float32)
    return x


def index_keys(seed: int, layer: int, b: int, t0: int, t1: int, planted, u, g: Geometry = GEOM,
               chunk: int = 1 << 16):
    """Quantised index keys of tokens [t0, t1): (codes u8 [n][64], scale bits u16 [n])."""
    codes = np.empty((t1 - t0, g.idx_dim), np.uint8)
    sig = np.empty(t1 - t0, np.uint16)
    for a in range(t0, t1, chunk):
        e = min(a + chunk, t1)
        c, s = quantise_rows(index_key_values(seed, layer, b, a, e, planted, u, g))
        codes[a - t0:e - t0] = c
        sig[a - t0:e - t0] = s
    return codes, sig


# ------------------------------------------------------------------ KV rows

def kv_rows(seed: int, layer: int, slots, g: Geometry = GEOM):
    """bf16 bits [len(slots)][row_elems] of the given physical slots."""
    s = np.asarray(slots, dtype=np.uint64)
    n = s[:, None] * np.uint64(g.row_elems) + np.arange(g.row_elems, dtype=np.uint64)[None, :]
    return f32_to_bf16_bits(normals(stream_key(seed, T_KV, layer), n))


# ------------------------------------------------------------- page tables

@dataclass
class Layout:
    """Host-side description of one batch: lengths, index-row offsets and the
    page table (shared by all layers)."""
    ctx: np.ndarray          # int64 [B]
    row0: np.ndarray         # int64 [B] first index row of each sequence
    n_rows: int              # total index rows per layer
    pt: np.ndarray           # int32 [B][pt_stride]
    n_slots: int
    planted: dict = field(default_factory=dict)   # (layer, b) -> int32 blocks


def make_layout(wl: Workload, g: Geometry = GEOM) -> Layout:
    ctx = ctx_lengths(wl)
    B = wl.batch
    row0 = np.zeros(B, np.int64)
    row0[1:] = np.cumsum(ctx)[:-1]
    n_rows = int(ctx.sum())
    stride = int(ctx.max())
    pt = np.full((B, stride), -1, np.int32)
    rng = np.random.Generator(np.random.PCG64([wl.seed, 303]))
    if wl.name == "tiny-4k":
        # identity plus a seeded random permutation of the physical slots
        n_slots = int(ctx[0])
        pt[0, :n_slots] = rng.permutation(n_slots).astype(np.int32)
    elif wl.tail_tokens > 0:
        # shared slot pool: disjoint draws for the body, plus a per-sequence ring
        # of tail_tokens slots that the last tail_tokens tokens map onto
        body = np.maximum(ctx - wl.tail_tokens, 0)
        n_body = int(body.sum())
        n_slots = n_body + B * wl.tail_tokens
        perm = rng.permutation(n_body).astype(np.int32)
        off = 0
        for b in range(B):
            L = int(ctx[b])
            nb = int(body[b])
            pt[b, :nb] = perm[off:off + nb]
            off += nb
            ring = n_body + b * wl.tail_tokens
            t = np.arange(nb, L)
            pt[b, nb:L] = (ring + (t % wl.tail_tokens)).astype(np.int32)
    else:
        # a seeded shuffle of the whole slot pool
        n_slots = n_rows
        perm = rng.permutation(n_slots).astype(np.int32)
        for b in range(B):
            pt[b, :ctx[b]] = perm[row0[b]:row0[b] + ctx[b]]
    lay = Layout(ctx, row0, n_rows, pt, n_slots)
    for layer in range(wl.layers):
        for b in range(B):
            lay.planted[(layer, b)] = planted_blocks(wl, layer, b, int(ctx[b]), g)
    return lay


@dataclass
class HostInputs:
    """Everything small, generated on the host; the big tensors (index keys and
    KV pools) are generated per sequence/slot on demand or filled on the GPU."""
    wl: Workload
    lay: Layout
    q_idx: np.ndarray   # u16 [layers][B][4][64]
    w: np.ndarray       # f32 [layers][B][4]
    q: np.ndarray       # u16 [layers][B][16][256]
    u: np.ndarray       # f32 [layers][B][64]


def host_inputs(wl: Workload, g: Geometry = GEOM) -> HostInputs:
    lay = make_layout(wl, g)
    B = wl.batch
    q_idx = np.stack([q_idx_bits(wl.seed, l, B, g) for l in range(wl.layers)])
    w = np.stack([w_idx(wl.seed, l, B, g) for l in range(wl.layers)])
    q = np.stack([q_bits(wl.seed, l, B, g) for l in range(wl.layers)])
    u = np.stack([np.stack([plant_direction(q_idx[l, b], w[l, b]) for b in range(B)])
                  for l in range(wl.layers)])
    return HostInputs(wl, lay, q_idx, w, q, u)


def host_index_layer(hi: HostInputs, layer: int, g: Geometry = GEOM):
    """Index keys of every sequence of one layer, packed by row0: (u8 [rows][64], u16 [rows])."""
    codes = np.empty((hi.lay.n_rows, g.idx_dim), np.uint8)
    sig = np.empty(hi.lay.n_rows, np.uint16)
    for b in range(hi.wl.batch):
        L = int(hi.lay.ctx[b])
        r0 = int(hi.lay.row0[b])
        c, s = index_keys(hi.wl.seed, layer, b, 0, L, hi.lay.planted[(layer, b)], hi.u[layer, b], g)
        codes[r0:r0 + L] = c
        sig[r0:r0 + L] = s
    return codes, sig


def host_pool_layer(hi: HostInputs, layer: int, g: Geometry = GEOM, chunk: int = 1 << 14):
    """The whole KV pool of one layer on the host, bf16 bits [n_slots][row_elems]."""
    out = np.empty((hi.lay.n_slots, g.row_elems), np.uint16)
    for a in range(0, hi.lay.n_slots, chunk):
        e = min(a + chunk, hi.lay.n_slots)
        out[a:e] = kv_rows(hi.wl.seed, layer, np.arange(a, e), g)
    return out


# ------------------------------------------------------------ decode steps

def step_queries(wl: Workload, hi: HostInputs, variant: int, g: Geometry = GEOM):
    """Queries of decode step `variant` (for workloads that run many steps):
    indexer queries = bf16(q_idx + drift * N(0,1)), noise from stream
    (seed, T_DRIFT, layer) at counters offset by the variant, so consecutive
    steps select overlapping token sets; attention queries are fresh N(0,1)
    draws from stream (seed, T_STEP_Q, layer). Returns (q_idx bits
    [layers][B][4][64], q bits [layers][B][16][256])."""
    B = wl.batch
    nqi = B * g.idx_heads * g.idx_dim
    nq = B * g.n_q_heads * g.head_dim
    qi, qq = [], []
    for l in range(wl.layers):
        noise = normals(stream_key(wl.seed, T_DRIFT, l), np.arange(nqi, dtype=np.uint64) + np.uint64(variant * nqi))
        base = bf16_bits_to_f32(hi.q_idx[l]).reshape(-1)
        qi.append(f32_to_bf16_bits((base + np.float32(wl.drift) * noise).astype(np.float32))
                  .reshape(B, g.idx_heads, g.idx_dim))
        v = normals(stream_key(wl.seed, T_STEP_Q, l), np.arange(nq, dtype=np.uint64) + np.uint64(variant * nq))
        qq.append(f32_to_bf16_bits(v).reshape(B, g.n_q_heads, g.head_dim))
    return np.stack(qi), np.stack(qq)
