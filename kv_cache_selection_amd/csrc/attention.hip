// attention.hip -- split-K GQA decode attention over the selected rows and the
// log-sum-exp merge of the splits.
//
// For query head h with KV head g = h / 8 and the selected tokens T:
//     z_t = sm_scale * (q_h . K_{g,t}),   out_h = sum_t softmax(z)_t V_{g,t}
// (the attention the article's "fast path" computes, restricted to the
// gathered set). The tokens are split into chunks of kTPS = 128; a workgroup
// (split s, KV head g, sequence b, layer of the launch) attends the 8 query
// heads of g over its chunk, one wave per 32 tokens, and writes the
// normalised partial output and its log-sum-exp; the merge kernel combines
// the splits exactly: out = sum_s e^{lse_s - LSE} O_s.
//
// Per wave (two tiles of 16 tokens):
//  - all K and V rows of both tiles are requested before the first multiply;
//  - QK^T on the matrix cores: v_mfma_f32_16x16x32_bf16 with A = the 8 query
//    heads (rows 8..15 zero) and B = 32 dims x 16 tokens read straight from
//    the KV rows (each lane loads 16 contiguous bytes of one token's K);
//  - one softmax over the wave's 32 tokens in fp32, the statistics reduced
//    across the 16 lanes that hold one head's scores with DPP row operations;
//  - PV on the matrix cores as well: the V rows go through LDS, where
//    ds_read_b64_tr_b16 reads them transposed (k = tokens), and P enters as
//    an exact bf16 high part plus a bf16 remainder (16 mantissa bits).
// The four waves of a workgroup then merge their partial states in LDS.
//
// Rows come either from the staging area (qsa_sparse_decode, the pinned-host
// path) or straight from the KV pool through the page table (the gather is
// fused into the attention when the pool is in HBM). One launch may cover
// several layers: their pointers travel in the kernel arguments.
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 16;                          // tokens per MFMA tile
constexpr int kTiles = 2;                          // tiles per wave
constexpr int kWaveTok = kTile * kTiles;           // 32
static_assert(kWaves * kWaveTok == kTPS, "tokens per split");
constexpr int kKBytes = kDh * 2;                   // 512 bytes of K (or V) per head per row
// A wave's V tile in LDS: 16 token rows of 512 bytes, 32 bytes of padding
// between rows so that the transposing reads of 16 rows hit distinct banks.
constexpr int kVPitch = kKBytes + 32;
constexpr int kVTileBytes = kWaveTok * kVPitch;    // a wave's 32 rows: 17408
constexpr int kOBytes = kWaves * kGroup * kDh * 4; // per-wave partial outputs for the merge (32 KB)
constexpr int kSmemBytes = kWaves * kVTileBytes > kOBytes ? kWaves * kVTileBytes : kOBytes;

// Max / sum over the 16 lanes of a DPP row (lanes 16r .. 16r + 15): swaps
// within pairs and quads, then the half-row and row mirrors.
template <bool kMax>
__device__ __forceinline__ float row16_reduce(float x)
{
    auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));  // quad_perm 1,0,3,2
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));  // quad_perm 2,3,0,1
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false))); // row_half_mirror
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false))); // row_mirror
    return x;
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Grid (n_split, kHkv * layers, B): workgroup (split s, KV head g of layer ly,
// sequence b) with blockIdx.y = g + kHkv * ly.
template <bool kPaged, int N>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(const AttnLayersT<N> Ls, int64_t pt_stride, int max_ctx,
                                                              int budget_blocks, int budget_tokens, float sm_scale,
                                                              int n_split)
{
    const int ly = blockIdx.y / kHkv;
    const uint16_t *__restrict__ q = Ls.q[ly];
    const uint8_t *__restrict__ rows = Ls.rows[ly];
    const int32_t *__restrict__ pt = Ls.pt[ly];
    const int64_t n_slots = Ls.n_slots[ly];
    const int32_t *__restrict__ sel = Ls.sel[ly];
    const int32_t *__restrict__ n_tok = Ls.n_tok[ly];
    float *__restrict__ part_o = Ls.part_o[ly];
    float *__restrict__ part_lse = Ls.part_lse[ly];
    __shared__ __attribute__((aligned(16))) float ps[kWaves][kGroup][kWaveTok];  // the wave's probabilities
    __shared__ float sstat[kWaves][kGroup][2];      // per-wave (max, sum) for the workgroup merge
    __shared__ float swt[kWaves][kGroup];           // per-wave weights exp(m_w - M) of each head
    __shared__ float sden[kGroup];                  // each head's normaliser
    // V tiles during the token loop, then the per-wave partial outputs
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];

    const int s = blockIdx.x;
    const int g = blockIdx.y % kHkv;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int split_p0 = s * kTPS;
    const int wave_p0 = split_p0 + wave * kWaveTok;
    const int arow = lane & 15;
    const int kofs = 8 * (lane >> 4);

    // Everything that does not depend on the token count is requested at
    // once: the count, the query, and each lane's row for its K token (lane
    // l holds token l & 15 of each tile). On the paged path the row is the
    // page-table slot of the selected token; indices are clamped so that
    // every read stays inside its buffer before the count is known.
    // The loads are unconditional (selects come after them), so that the
    // compiler can count them: the selection entries of both tiles and the
    // query go out together, then the page-table slots of both tiles.
    int nt = n_tok[b];
    int64_t row_k[kTiles];
    int ptok[kTiles], stok[kTiles];
#pragma unroll
    for (int i = 0; i < kTiles; i++) {
        const int p = min(wave_p0 + kTile * i + arow, budget_tokens - 1);
        ptok[i] = p;
        if (kPaged)
            stok[i] = sel[(int64_t)b * budget_blocks + (p >> 2)];
    }
    // A operand: lane holds row (lane & 15) = query head of group g, dims
    // 32kk + 8 (lane >> 4) .. +8 for MFMA kk. Rows 8..15 repeat rows 0..7;
    // their outputs land in lanes 32..63, which carry no head and are never
    // used.
    bf16x8 qa[kDh / 32];
    {
        const uint16_t *qr = q + ((int64_t)b * kHq + g * kGroup + (arow & 7)) * kDh + kofs;
#pragma unroll
        for (int kk = 0; kk < kDh / 32; kk++)
            qa[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qr + 32 * kk));
    }
    if (kPaged) {
        // token t of the selection; a block index outside the context (only
        // in entries past the count) reads slot 0. With no context the table
        // may be empty, so a selection entry is read instead.
        int32_t slot[kTiles];
        bool in[kTiles];
#pragma unroll
        for (int i = 0; i < kTiles; i++) {
            const int t = stok[i] * kBT + (ptok[i] & 3);
            in[i] = t >= 0 && max_ctx > 0;
            const int tc = min(max(t, 0), max_ctx - 1);
            const int32_t *src = max_ctx > 0 ? pt + (int64_t)b * pt_stride + tc : sel + (int64_t)b * budget_blocks;
            slot[i] = *src;
        }
        // both slots are used here, so both reads are issued before either
        // is waited for (not moved into the branches of the selects below)
        static_assert(kTiles == 2, "two tiles per wave");
        asm volatile("" : "+v"(slot[0]), "+v"(slot[1]));
#pragma unroll
        for (int i = 0; i < kTiles; i++)
            row_k[i] = in[i] ? safe_slot(slot[i], n_slots) : 0;
    } else {
#pragma unroll
        for (int i = 0; i < kTiles; i++)
            row_k[i] = (int64_t)b * budget_tokens + ptok[i];
    }

    nt = nt < 0 ? 0 : (nt > budget_tokens ? budget_tokens : nt);
    const int64_t part_base = ((int64_t)b * kHq + g * kGroup) * n_split + s;   // head g*8, split s
    if (split_p0 >= nt) {
        if (tid < kGroup)
            part_lse[part_base + (int64_t)tid * n_split] = -INFINITY;
        return;
    }

    // Softmax state of the wave: lane l holds heads 4 (l >> 4) + v (rows 8..15
    // of the MFMA tiles are padding, so lanes 32..63 carry no head). The
    // wave's 32 tokens are normalised together, so no running rescale.
    float m_run[4], l_run[4];
    // Output accumulators, the C tiles of PV: o[m][v] = head 4 (l >> 4) + v,
    // dim 16 m + (l & 15).
    f32x4 o[kDh / 16];
#pragma unroll
    for (int m = 0; m < kDh / 16; m++)
        o[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    uint8_t *vt = smem + wave * kVTileBytes;
    const int grp = lane >> 4;
    const int col = lane & 15;

    if (wave_p0 >= nt) {                            // uniform: no valid token in this wave
#pragma unroll
        for (int v = 0; v < 4; v++) {
            m_run[v] = -INFINITY;
            l_run[v] = 0.0f;
        }
    } else {
        // Request every row the wave needs before the first multiply: the K
        // rows of both tiles, then their V rows (the V rows of a tile's 16
        // tokens are the K rows held by lanes 0..15). Every request is made,
        // also for tokens past the count, whose row indices are clamped to
        // valid rows and whose scores and V rows are masked below; so the
        // compiler can count the requests, and QK^T and the softmax start as
        // soon as the K rows are in, while the V rows still arrive.
        u32x4 kd[kTiles][kDh / 32];
        u32x2 vd[kTiles][kTile];
#pragma unroll
        for (int i = 0; i < kTiles; i++) {
            const uint8_t *rk = rows + row_k[i] * kRowBytes + g * kKBytes + 2 * kofs;
#pragma unroll
            for (int kk = 0; kk < kDh / 32; kk++)
                kd[i][kk] = *reinterpret_cast<const u32x4 *>(rk + 64 * kk);
        }
#pragma unroll
        for (int i = 0; i < kTiles; i++) {
            const uint32_t rlo = (uint32_t)row_k[i], rhi = (uint32_t)(row_k[i] >> 32);
#pragma unroll
            for (int t = 0; t < kTile; t++) {
                // uniform across the wave: token wave_p0 + 16 i + t, whose row lane t holds
                const int64_t r = (int64_t)(((uint64_t)__builtin_amdgcn_readlane(rhi, t) << 32) |
                                            __builtin_amdgcn_readlane(rlo, t));
                vd[i][t] = *reinterpret_cast<const u32x2 *>(rows + r * kRowBytes + (kHkv + g) * kKBytes + 8 * lane);
            }
        }
        f32x4 acc[kTiles];
#pragma unroll
        for (int i = 0; i < kTiles; i++) {
            acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < kDh / 32; kk++)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], __builtin_bit_cast(bf16x8, kd[i][kk]),
                                                                 acc[i], 0, 0, 0);
        }
        // acc[i][v] = q_{4 (lane>>4) + v} . K_{token 16 i + (lane & 15)}.
#pragma unroll
        for (int v = 0; v < 4; v++) {
            float z[kTiles], mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < kTiles; i++) {
                z[i] = wave_p0 + kTile * i + col < nt ? acc[i][v] * sm_scale : -INFINITY;
                mx = fmaxf(mx, z[i]);
            }
            mx = row16_reduce<true>(mx);
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < kTiles; i++) {
                float e = (z[i] == -INFINITY) ? 0.0f : __expf(z[i] - mx);
                // Keep 16 mantissa bits (a bf16 head plus a bf16 remainder),
                // the precision PV uses, so that numerator and normaliser agree.
                const uint32_t hb = __float_as_uint(e) & 0xFFFF0000u;
                const uint32_t lb = __float_as_uint(e - __uint_as_float(hb)) & 0xFFFF0000u;
                e = __uint_as_float(hb) + __uint_as_float(lb);
                sum += e;
                if (lane < 32)
                    ps[wave][4 * grp + v][kTile * i + col] = e;
            }
            l_run[v] = row16_reduce<false>(sum);
            m_run[v] = mx;
        }
        // V rows of both tiles to LDS (row 16 i + t), zero past the count
#pragma unroll
        for (int i = 0; i < kTiles; i++)
#pragma unroll
            for (int t = 0; t < kTile; t++)
                *reinterpret_cast<u32x2 *>(vt + (kTile * i + t) * kVPitch + 8 * lane) =
                    wave_p0 + kTile * i + t < nt ? vd[i][t] : u32x2{0u, 0u};
        wave_lds_sync();

        // PV on the matrix cores, v_mfma_f32_16x16x32_bf16 per 16 dims:
        //  A = P (row = head `col`, k = tokens 8 grp .. +7) as its exact split
        //      into a bf16 high part and a bf16 remainder;
        //  B = V (k = tokens 8 grp .. +7, column = dim), read transposed from
        //      the rows in LDS, four tokens per read: in each group of 16
        //      lanes, lane j supplies the address of token row base + (j >> 2),
        //      dims 4 (j & 3) .. +3, and lane c receives dim c of the four rows.
        bf16x8 a_hi, a_lo;
        {
            uint32_t hi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
            if (col < kGroup) {
                const f32x4 p0 = *reinterpret_cast<const f32x4 *>(&ps[wave][col][8 * grp]);
                const f32x4 p1 = *reinterpret_cast<const f32x4 *>(&ps[wave][col][8 * grp + 4]);
                const float pv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const uint32_t h0 = __float_as_uint(pv[e]) & 0xFFFF0000u;
                    const uint32_t h1 = __float_as_uint(pv[e + 1]) & 0xFFFF0000u;
                    const uint32_t l0 = __float_as_uint(pv[e] - __uint_as_float(h0)) >> 16;
                    const uint32_t l1 = __float_as_uint(pv[e + 1] - __uint_as_float(h1)) & 0xFFFF0000u;
                    hi[e >> 1] = (h0 >> 16) | h1;
                    lo[e >> 1] = l0 | l1;
                }
            }
            a_hi = __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
            a_lo = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
        }
        const uint8_t *vrd = vt + (8 * grp + (col >> 2)) * kVPitch + 8 * (col & 3);
#pragma unroll
        for (int m = 0; m < kDh / 16; m++) {
            const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(vrd + 32 * m));
            const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(vrd + 4 * kVPitch + 32 * m));
            const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
            o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, bv, o[m], 0, 0, 0);
            o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, bv, o[m], 0, 0, 0);
        }
    }

    // Workgroup merge of the four waves' states (the V tiles' LDS is reused):
    // each wave's accumulators go to LDS as [dim][head], 16 bytes (4 heads of
    // one dim) per store; 8 threads then work out each head's wave weights
    // f_w = exp(m_w - M), normaliser and LSE once, and every thread combines
    // one dim for the 8 heads.
    __syncthreads();
    float(*sod)[kDh][kGroup] = reinterpret_cast<float(*)[kDh][kGroup]>(smem);
    if (lane < 32) {
#pragma unroll
        for (int m = 0; m < kDh / 16; m++)
            *reinterpret_cast<f32x4 *>(&sod[wave][16 * m + col][4 * grp]) = o[m];
    }
    if (lane < 32 && (lane & 15) == 0) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            sstat[wave][4 * (lane >> 4) + v][0] = m_run[v];
            sstat[wave][4 * (lane >> 4) + v][1] = l_run[v];
        }
    }
    __syncthreads();
    if (tid < kGroup) {
        const int h = tid;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++)
            M = fmaxf(M, sstat[w][h][0]);
        float den = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float mw = sstat[w][h][0];
            const float f = (mw == -INFINITY) ? 0.0f : __expf(mw - M);
            swt[w][h] = f;
            den += f * sstat[w][h][1];
        }
        sden[h] = den;
        part_lse[part_base + (int64_t)h * n_split] = M + logf(den);
    }
    __syncthreads();
    for (int d = tid; d < kDh; d += kThreads) {
        float acc[kGroup];
#pragma unroll
        for (int h = 0; h < kGroup; h++)
            acc[h] = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(&sod[w][d][0]);
            const f32x4 c = *reinterpret_cast<const f32x4 *>(&sod[w][d][4]);
#pragma unroll
            for (int h = 0; h < 4; h++) {
                acc[h] = fmaf(swt[w][h], a[h], acc[h]);
                acc[4 + h] = fmaf(swt[w][4 + h], c[h], acc[4 + h]);
            }
        }
#pragma unroll
        for (int h = 0; h < kGroup; h++)
            part_o[(part_base + (int64_t)h * n_split) * kDh + d] = acc[h] / sden[h];
    }
}

constexpr int kMergeUnroll = 16;

// One workgroup per (sequence, head) and layer (grid (B * kHq, layers));
// thread d owns output dim d. Every thread reads the (uniform) split LSEs
// itself and its column of partial outputs in the same batch, so the whole
// merge is one round of loads: for each batch of splits, the running max is
// raised and the sums rescaled.
template <int N>
__global__ __launch_bounds__(kDh) void merge_kernel(const AttnLayersT<N> Ls, int n_split)
{
    const float *__restrict__ part_o = Ls.part_o[blockIdx.y];
    const float *__restrict__ part_lse = Ls.part_lse[blockIdx.y];
    float *__restrict__ out = Ls.out[blockIdx.y];
    const int bh = blockIdx.x;              // b * kHq + h
    const int tid = threadIdx.x;
    const float *lse = part_lse + (int64_t)bh * n_split;
    const float *col = part_o + (int64_t)bh * n_split * kDh + tid;
    float M = -INFINITY, acc = 0.0f, den = 0.0f;
    for (int s0 = 0; s0 < n_split; s0 += kMergeUnroll) {
        float ls[kMergeUnroll], x[kMergeUnroll];
#pragma unroll
        for (int u = 0; u < kMergeUnroll; u++) {
            const bool in = s0 + u < n_split;
            ls[u] = in ? lse[s0 + u] : -INFINITY;
            x[u] = in ? col[(int64_t)(s0 + u) * kDh] : 0.0f;
        }
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < kMergeUnroll; u++)
            mb = fmaxf(mb, ls[u]);
        if (mb == -INFINITY)
            continue;                       // uniform: every split of the batch is empty
        const float Mn = fmaxf(M, mb);
        const float r = __expf(M - Mn);     // 0 while M is still -inf
        acc *= r;
        den *= r;
#pragma unroll
        for (int u = 0; u < kMergeUnroll; u++) {
            const float ws = ls[u] == -INFINITY ? 0.0f : __expf(ls[u] - Mn);
            den += ws;
            // empty splits hold stale data: select, not multiply
            acc = ws != 0.0f ? fmaf(ws, x[u], acc) : acc;
        }
        M = Mn;
    }
    out[(int64_t)bh * kDh + tid] = den > 0.0f ? acc / den : 0.0f;
}

} // namespace

template <int N>
static hipError_t launch_attention_n(bool paged, const AttnLayersT<N> &L, int n_layers, int64_t pt_stride,
                                     int max_ctx, int batch, int budget_blocks, int budget_tokens, float sm_scale,
                                     int n_split, hipStream_t s)
{
    dim3 grid((unsigned)n_split, (unsigned)(kHkv * n_layers), (unsigned)batch);
    if (paged)
        hipLaunchKernelGGL((attn_split_kernel<true, N>), grid, dim3(kThreads), 0, s, L, pt_stride, max_ctx,
                           budget_blocks, budget_tokens, sm_scale, n_split);
    else
        hipLaunchKernelGGL((attn_split_kernel<false, N>), grid, dim3(kThreads), 0, s, L, pt_stride, max_ctx,
                           budget_blocks, budget_tokens, sm_scale, n_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((merge_kernel<N>), dim3((unsigned)(batch * kHq), (unsigned)n_layers), dim3(kDh), 0, s, L,
                       n_split);
    return hipGetLastError();
}

hipError_t launch_attention_layers(bool paged, const AttnLayers &L, int n_layers, int64_t pt_stride, int max_ctx,
                                   int batch, int budget_blocks, int budget_tokens, float sm_scale, int n_split,
                                   hipStream_t s)
{
    if (n_layers < 1 || n_layers > kMaxChainLayers)
        return hipErrorInvalidValue;
    if (n_layers > 1)
        return launch_attention_n(paged, L, n_layers, pt_stride, max_ctx, batch, budget_blocks, budget_tokens,
                                  sm_scale, n_split, s);
    const AttnLayersT<1> L1 = {{L.q[0]},     {L.rows[0]},   {L.pt[0]},       {L.n_slots[0]}, {L.sel[0]},
                               {L.n_tok[0]}, {L.part_o[0]}, {L.part_lse[0]}, {L.out[0]}};
    return launch_attention_n(paged, L1, 1, pt_stride, max_ctx, batch, budget_blocks, budget_tokens, sm_scale,
                              n_split, s);
}

hipError_t launch_attention_staged(const uint16_t *q, const void *kv, const int32_t *n_tok, int batch,
                                   int budget_tokens, float sm_scale, const AttnWs &ws, float *out, hipStream_t s)
{
    AttnLayers L = {};
    L.q[0] = q;
    L.rows[0] = static_cast<const uint8_t *>(kv);
    L.n_tok[0] = n_tok;
    L.part_o[0] = ws.part_o;
    L.part_lse[0] = ws.part_lse;
    L.out[0] = out;
    return launch_attention_layers(false, L, 1, 0, 0, batch, 0, budget_tokens, sm_scale, ws.n_split, s);
}

hipError_t launch_attention_paged(const uint16_t *q, const void *pool, const int32_t *pt, int64_t pt_stride,
                                  int64_t n_slots, const int32_t *sel, const int32_t *n_tok, const int32_t *ctx_len,
                                  int max_ctx, int batch, int budget_blocks, int budget_tokens, float sm_scale,
                                  const AttnWs &ws, float *out, hipStream_t s)
{
    (void)ctx_len;
    AttnLayers L = {};
    L.q[0] = q;
    L.rows[0] = static_cast<const uint8_t *>(pool);
    L.pt[0] = pt;
    L.n_slots[0] = n_slots;
    L.sel[0] = sel;
    L.n_tok[0] = n_tok;
    L.part_o[0] = ws.part_o;
    L.part_lse[0] = ws.part_lse;
    L.out[0] = out;
    return launch_attention_layers(true, L, 1, pt_stride, max_ctx, batch, budget_blocks, budget_tokens, sm_scale,
                                   ws.n_split, s);
}

} // namespace qsa
