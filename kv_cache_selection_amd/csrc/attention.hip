// attention.hip -- split-K GQA decode attention over the selected rows and the
// log-sum-exp merge of the splits.
//
// For query head h with KV head g = h / 8 and the selected tokens T:
//     z_t = sm_scale * (q_h . K_{g,t}),   out_h = sum_t softmax(z)_t V_{g,t}
// (the attention the article's "fast path" computes, restricted to the
// gathered set). The tokens are split into chunks of kTPS = 128; a workgroup
// (sequence b, KV head g, split s) attends the 8 query heads of g over its
// chunk, one wave per 32 tokens, and writes the normalised partial output and
// its log-sum-exp; the merge kernel combines the splits exactly:
// out = sum_s e^{lse_s - LSE} O_s.
//
// Per wave and tile of 16 tokens:
//  - QK^T on the matrix cores: v_mfma_f32_16x16x32_bf16 with A = the 8 query
//    heads (rows 8..15 zero) and B = 32 dims x 16 tokens read straight from
//    the KV rows (each lane loads 16 contiguous bytes of one token's K);
//  - online softmax over the tile in fp32, statistics reduced across the 16
//    lanes that hold one head's scores;
//  - PV on the VALU in fp32: each lane owns 4 of the 256 dims for all 8
//    heads and streams the tile's V rows (8 contiguous bytes per lane and
//    token), the tile's probabilities broadcast through LDS.
// The four waves of a workgroup merge their partial states in LDS. All rows
// of a wave's two tiles are requested before the first multiply.
//
// Rows come either from the staging area (qsa_sparse_decode, offload path) or
// straight from the KV pool through the page table (gather fused into the
// attention when the pool is in HBM).
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 16;                          // tokens per MFMA tile
constexpr int kTiles = 2;                          // tiles per wave
constexpr int kWaveTok = kTile * kTiles;           // 32
static_assert(kWaves * kWaveTok == kTPS, "tokens per split");
constexpr int kKBytes = kDh * 2;                   // 512 bytes of K (or V) per head per row

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool kPaged>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ rows, const int32_t *__restrict__ pt,
    int64_t pt_stride, int64_t n_slots, const int32_t *__restrict__ sel, const int32_t *__restrict__ n_tok,
    int max_ctx, int budget_blocks, int budget_tokens, float sm_scale, float *__restrict__ part_o,
    float *__restrict__ part_lse, int n_split)
{
    __shared__ float ps[kWaves][kGroup][kTile];     // probabilities of the wave's current tile
    __shared__ float salpha[kWaves][kGroup];        // per-head rescale of the wave's running output
    __shared__ float sstat[kWaves][kGroup][2];      // per-wave (max, sum) for the workgroup merge
    __shared__ float so[kWaves][kGroup][kDh];       // per-wave partial outputs (32 KB)

    const int s = blockIdx.x;
    const int g = blockIdx.y;
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
    int nt = n_tok[b];
    int64_t row_k[kTiles];
#pragma unroll
    for (int i = 0; i < kTiles; i++) {
        int p = wave_p0 + kTile * i + arow;
        p = p < budget_tokens ? p : budget_tokens - 1;
        if (kPaged) {
            int t = sel[(int64_t)b * budget_blocks + (p >> 2)] * kBT + (p & 3);
            t = t < max_ctx ? t : max_ctx - 1;
            row_k[i] = t >= 0 ? safe_slot(pt[(int64_t)b * pt_stride + t], n_slots) : 0;
        } else {
            row_k[i] = (int64_t)b * budget_tokens + p;
        }
    }
    // A operand: lane holds row (lane & 15) = query head of group g (rows 8..15
    // zero), dims 32kk + 8 (lane >> 4) .. +8 for MFMA kk.
    bf16x8 qa[kDh / 32];
    {
        const uint16_t *qr = q + ((int64_t)b * kHq + g * kGroup + (arow & 7)) * kDh + kofs;
#pragma unroll
        for (int kk = 0; kk < kDh / 32; kk++) {
            const u32x4 v = arow < kGroup ? *reinterpret_cast<const u32x4 *>(qr + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
            qa[kk] = __builtin_bit_cast(bf16x8, v);
        }
    }

    nt = nt < 0 ? 0 : (nt > budget_tokens ? budget_tokens : nt);
    const int64_t part_base = ((int64_t)b * kHq + g * kGroup) * n_split + s;   // head g*8, split s
    if (split_p0 >= nt) {
        if (tid < kGroup)
            part_lse[part_base + (int64_t)tid * n_split] = -INFINITY;
        return;
    }

    // Request every row the wave needs before the first multiply. The V rows
    // of a tile's 16 tokens are the K rows held by lanes 0..15.
    u32x4 kd[kTiles][kDh / 32];
    u32x2 vd[kTiles][kTile];
#pragma unroll
    for (int i = 0; i < kTiles; i++) {
        const int pt0 = wave_p0 + kTile * i;
        if (pt0 + arow < nt) {
            const uint8_t *rk = rows + row_k[i] * kRowBytes + g * kKBytes + 2 * kofs;
#pragma unroll
            for (int kk = 0; kk < kDh / 32; kk++)
                kd[i][kk] = *reinterpret_cast<const u32x4 *>(rk + 64 * kk);
        } else {
#pragma unroll
            for (int kk = 0; kk < kDh / 32; kk++)
                kd[i][kk] = u32x4{0u, 0u, 0u, 0u};
        }
        const uint32_t rlo = (uint32_t)row_k[i], rhi = (uint32_t)(row_k[i] >> 32);
#pragma unroll
        for (int t = 0; t < kTile; t++) {
            // uniform across the wave: token pt0 + t, whose row lane t holds
            const int64_t r = (int64_t)(((uint64_t)__builtin_amdgcn_readlane(rhi, t) << 32) |
                                        __builtin_amdgcn_readlane(rlo, t));
            vd[i][t] = pt0 + t < nt
                           ? *reinterpret_cast<const u32x2 *>(rows + r * kRowBytes + (kHkv + g) * kKBytes + 8 * lane)
                           : u32x2{0u, 0u};
        }
    }

    // Running softmax state: lanes 0..31 hold heads 4 (lane >> 4) + v.
    float m_run[4], l_run[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        m_run[v] = -INFINITY;
        l_run[v] = 0.0f;
    }
    float o[kGroup][4];                             // this lane's 4 dims of every head
#pragma unroll
    for (int h = 0; h < kGroup; h++)
#pragma unroll
        for (int c = 0; c < 4; c++)
            o[h][c] = 0.0f;

#pragma unroll
    for (int i = 0; i < kTiles; i++) {
        const int pt0 = wave_p0 + kTile * i;
        if (pt0 >= nt)
            break;                                  // uniform: no valid token left in this wave
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < kDh / 32; kk++)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], __builtin_bit_cast(bf16x8, kd[i][kk]), acc, 0, 0,
                                                          0);
        // acc[v] = q_{4 (lane>>4) + v} . K_{token lane & 15}; rows >= 8 are padding.
        const bool tok_ok = pt0 + (lane & 15) < nt;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const float z = tok_ok ? acc[v] * sm_scale : -INFINITY;
            float mx = z;
#pragma unroll
            for (int o2 = 8; o2 >= 1; o2 >>= 1)
                mx = fmaxf(mx, __shfl_xor(mx, o2, 16));
            const float mn = fmaxf(m_run[v], mx);
            const float alpha = (mn == -INFINITY) ? 1.0f : __expf(m_run[v] - mn);
            const float e = (z == -INFINITY) ? 0.0f : __expf(z - mn);
            float sum = e;
#pragma unroll
            for (int o2 = 8; o2 >= 1; o2 >>= 1)
                sum += __shfl_xor(sum, o2, 16);
            l_run[v] = l_run[v] * alpha + sum;
            m_run[v] = mn;
            if (lane < 32) {
                const int h = 4 * (lane >> 4) + v;
                ps[wave][h][lane & 15] = e;
                if ((lane & 15) == 0)
                    salpha[wave][h] = alpha;
            }
        }
        wave_lds_sync();

        // PV: rescale, then accumulate the tile's 16 rows.
#pragma unroll
        for (int h = 0; h < kGroup; h++) {
            const float a = salpha[wave][h];
#pragma unroll
            for (int c = 0; c < 4; c++)
                o[h][c] *= a;
        }
#pragma unroll
        for (int t = 0; t < kTile; t++) {
            const u32x2 w = vd[i][t];
            const float v0 = __uint_as_float(w.x << 16), v1 = __uint_as_float(w.x & 0xFFFF0000u);
            const float v2 = __uint_as_float(w.y << 16), v3 = __uint_as_float(w.y & 0xFFFF0000u);
#pragma unroll
            for (int h = 0; h < kGroup; h++) {
                const float p = ps[wave][h][t];
                o[h][0] = fmaf(p, v0, o[h][0]);
                o[h][1] = fmaf(p, v1, o[h][1]);
                o[h][2] = fmaf(p, v2, o[h][2]);
                o[h][3] = fmaf(p, v3, o[h][3]);
            }
        }
        wave_lds_sync();
    }

    // Workgroup merge of the four waves' states.
#pragma unroll
    for (int h = 0; h < kGroup; h++)
        *reinterpret_cast<f32x4 *>(&so[wave][h][4 * lane]) = f32x4{o[h][0], o[h][1], o[h][2], o[h][3]};
    if (lane < 32 && (lane & 15) == 0) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            sstat[wave][4 * (lane >> 4) + v][0] = m_run[v];
            sstat[wave][4 * (lane >> 4) + v][1] = l_run[v];
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kGroup; h++) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++)
            M = fmaxf(M, sstat[w][h][0]);
        float acc = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float mw = sstat[w][h][0];
            const float f = (mw == -INFINITY) ? 0.0f : __expf(mw - M);
            den += f * sstat[w][h][1];
            acc = fmaf(f, so[w][h][tid], acc);
        }
        part_o[(part_base + (int64_t)h * n_split) * kDh + tid] = acc / den;
        if (tid == 0)
            part_lse[part_base + (int64_t)h * n_split] = M + logf(den);
    }
}

constexpr int kMaxSplit = kMaxBudget / kTPS;
constexpr int kMergeUnroll = 16;

// One workgroup per (sequence, head); thread d owns output dim d. The split
// weights e^{lse_s - max} are computed once into LDS, then every thread sums
// its column with all loads of a batch of splits in flight.
__global__ __launch_bounds__(kDh) void merge_kernel(const float *__restrict__ part_o,
                                                    const float *__restrict__ part_lse, int n_split,
                                                    float *__restrict__ out)
{
    __shared__ float wgt[kMaxSplit];
    __shared__ float red[kDh / 64];
    const int bh = blockIdx.x;              // b * kHq + h
    const int tid = threadIdx.x;
    const float *lse = part_lse + (int64_t)bh * n_split;
    const float ls = tid < n_split ? lse[tid] : -INFINITY;
    float m = ls;
    for (int o = 32; o >= 1; o >>= 1)
        m = fmaxf(m, __shfl_xor(m, o));
    if ((tid & 63) == 0)
        red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (tid < n_split)
        wgt[tid] = (m == -INFINITY || ls == -INFINITY) ? 0.0f : __expf(ls - m);
    __syncthreads();
    float acc = 0.0f, den = 0.0f;
    if (m != -INFINITY) {
        const float *col = part_o + (int64_t)bh * n_split * kDh + tid;
        for (int s0 = 0; s0 < n_split; s0 += kMergeUnroll) {
            float x[kMergeUnroll];
#pragma unroll
            for (int u = 0; u < kMergeUnroll; u++)
                x[u] = s0 + u < n_split ? col[(int64_t)(s0 + u) * kDh] : 0.0f;
#pragma unroll
            for (int u = 0; u < kMergeUnroll; u++) {
                if (s0 + u < n_split) {
                    const float ws = wgt[s0 + u];
                    den += ws;
                    // empty splits hold stale data: select, not multiply
                    acc = ws != 0.0f ? fmaf(ws, x[u], acc) : acc;
                }
            }
        }
        acc /= den;
    }
    out[(int64_t)bh * kDh + tid] = acc;
}

} // namespace

static hipError_t launch_merge(const AttnWs &ws, int batch, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(batch * kHq)), dim3(kDh), 0, s, ws.part_o, ws.part_lse,
                       ws.n_split, out);
    return hipGetLastError();
}

hipError_t launch_attention_staged(const uint16_t *q, const void *kv, const int32_t *n_tok, int batch,
                                   int budget_tokens, float sm_scale, const AttnWs &ws, float *out, hipStream_t s)
{
    dim3 grid((unsigned)ws.n_split, (unsigned)kHkv, (unsigned)batch);
    hipLaunchKernelGGL((attn_split_kernel<false>), grid, dim3(kThreads), 0, s, q,
                       static_cast<const uint8_t *>(kv), nullptr, 0, 0, nullptr, n_tok, 0, 0, budget_tokens, sm_scale,
                       ws.part_o, ws.part_lse, ws.n_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_merge(ws, batch, out, s);
}

hipError_t launch_attention_paged(const uint16_t *q, const void *pool, const int32_t *pt, int64_t pt_stride,
                                  int64_t n_slots, const int32_t *sel, const int32_t *n_tok, const int32_t *ctx_len,
                                  int max_ctx, int batch, int budget_blocks, int budget_tokens, float sm_scale,
                                  const AttnWs &ws, float *out, hipStream_t s)
{
    dim3 grid((unsigned)ws.n_split, (unsigned)kHkv, (unsigned)batch);
    hipLaunchKernelGGL((attn_split_kernel<true>), grid, dim3(kThreads), 0, s, q,
                       static_cast<const uint8_t *>(pool), pt, pt_stride, n_slots, sel, n_tok, max_ctx, budget_blocks,
                       budget_tokens, sm_scale, ws.part_o, ws.part_lse, ws.n_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_merge(ws, batch, out, s);
}

} // namespace qsa
