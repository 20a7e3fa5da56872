// attention.hip -- split-K GQA decode attention over the selected rows and the
// log-sum-exp merge of the splits.
//
// For query head h with KV head g = h / 8 and the selected tokens T:
//     z_t = sm_scale * (q_h . K_{g,t}),   out_h = sum_t softmax(z)_t V_{g,t}
// (the attention the article's "fast path" computes, restricted to the
// gathered set). The tokens are split into chunks of kTPS; each workgroup
// (sequence b, KV head g, split s) attends the 8 query heads of g over its
// chunk and writes the normalised partial output and its log-sum-exp; the
// merge combines the splits exactly: out = sum_s e^{lse_s - LSE} O_s.
//
// Rows come either from the staging area (qsa_sparse_decode, offload path) or
// straight from the KV pool through the page table (gather fused into the
// attention when the pool is in HBM).
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 256;
constexpr int kKStride = kDh / 2 + 1;      // dwords per K row in LDS (+1 pad: conflict-free columns)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <bool kPaged>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ rows, const int32_t *__restrict__ pt,
    int64_t pt_stride, int64_t n_slots, const int32_t *__restrict__ sel, const int32_t *__restrict__ n_tok,
    const int32_t *__restrict__ ctx_len, int max_ctx, int budget_blocks, int budget_tokens, float sm_scale,
    float *__restrict__ part_o, float *__restrict__ part_lse, int n_split)
{
    __shared__ float qs[kGroup][kDh];                   // 8 KB
    __shared__ uint32_t ks[kTPS][kKStride];             // 33 KB
    __shared__ uint32_t vs[kTPS][kDh / 2];              // 32 KB
    __shared__ float ps[kGroup][kTPS];                  // 2 KB
    __shared__ float stat[kGroup][2];                   // max, sum

    const int s = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;

    int nt = n_tok[b];
    nt = nt < 0 ? 0 : (nt > budget_tokens ? budget_tokens : nt);
    const int p0 = s * kTPS;
    const int64_t part_base = ((int64_t)b * kHq + g * kGroup) * n_split + s;   // head g*8, split s
    if (p0 >= nt) {
        if (tid < kGroup)
            part_lse[part_base + (int64_t)tid * n_split] = -INFINITY;
        return;
    }
    const int cnt = min(kTPS, nt - p0);
    const int L = kPaged ? clamp_ctx(ctx_len[b], max_ctx) : 0;

    // q of the 8 heads of group g, as float.
    {
        const uint16_t *qg = q + ((int64_t)b * kHq + g * kGroup) * kDh;
        for (int i = tid; i < kGroup * kDh; i += kThreads)
            (&qs[0][0])[i] = __uint_as_float((uint32_t)qg[i] << 16);
    }
    // K and V of KV head g for the chunk's tokens: 32 pieces of 16 B each.
#pragma unroll
    for (int k = 0; k < (kTPS * 32) / kThreads; k++) {
        const int c = tid + k * kThreads;
        const int tok = c >> 5;
        const int piece = c & 31;
        uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
        if (tok < cnt) {
            const int p = p0 + tok;
            const uint8_t *row;
            if (kPaged) {
                const int j = sel[(int64_t)b * budget_blocks + (p >> 2)];
                const int t = j * kBT + (p & 3);
                const int64_t slot = safe_slot(pt[(int64_t)b * pt_stride + ((t >= 0 && t < L) ? t : 0)], n_slots);
                row = rows + slot * kRowBytes;
            } else {
                row = rows + ((int64_t)b * budget_tokens + p) * kRowBytes;
            }
            kv4 = *reinterpret_cast<const uint4 *>(row + g * (kDh * 2) + piece * 16);
            vv4 = *reinterpret_cast<const uint4 *>(row + (kHkv + g) * (kDh * 2) + piece * 16);
        }
        uint32_t *kd = &ks[tok][piece * 4];
        kd[0] = kv4.x;
        kd[1] = kv4.y;
        kd[2] = kv4.z;
        kd[3] = kv4.w;
        *reinterpret_cast<uint4 *>(&vs[tok][piece * 4]) = vv4;
    }
    __syncthreads();

    // Scores: thread -> head hl = tid / 32, tokens tl and tl + 32.
    const int hl = tid >> 5;
    const int tl = tid & 31;
    float z[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int tok = tl + 32 * u;
        float acc = 0.0f;
        const uint32_t *kr = ks[tok];
        const float *qh = qs[hl];
#pragma unroll 8
        for (int d2 = 0; d2 < kDh / 2; d2++) {
            const uint32_t w = kr[d2];
            acc = fmaf(qh[2 * d2], bf16_lo(w), acc);
            acc = fmaf(qh[2 * d2 + 1], bf16_hi(w), acc);
        }
        z[u] = tok < cnt ? acc * sm_scale : -INFINITY;
    }
    // Softmax statistics over the 64 tokens of head hl (32 lanes x 2 values).
    float m = fmaxf(z[0], z[1]);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1)
        m = fmaxf(m, __shfl_xor(m, o, 32));
    const float e0 = __expf(z[0] - m);
    const float e1 = __expf(z[1] - m);
    float l = e0 + e1;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1)
        l += __shfl_xor(l, o, 32);
    ps[hl][tl] = e0;
    ps[hl][tl + 32] = e1;
    if (tl == 0) {
        stat[hl][0] = m;
        stat[hl][1] = l;
    }
    __syncthreads();

    // PV: thread -> output dim d = tid, all 8 heads.
    float acc[kGroup];
#pragma unroll
    for (int h = 0; h < kGroup; h++)
        acc[h] = 0.0f;
    const uint16_t *vcol = reinterpret_cast<const uint16_t *>(&vs[0][0]) + tid;
    for (int tok = 0; tok < cnt; tok++) {
        const float v = __uint_as_float((uint32_t)vcol[tok * kDh] << 16);
#pragma unroll
        for (int h = 0; h < kGroup; h++)
            acc[h] = fmaf(ps[h][tok], v, acc[h]);
    }
#pragma unroll
    for (int h = 0; h < kGroup; h++) {
        const float lh = stat[h][1];
        part_o[(part_base + (int64_t)h * n_split) * kDh + tid] = acc[h] / lh;
        if (tid == 0)
            part_lse[part_base + (int64_t)h * n_split] = stat[h][0] + logf(lh);
    }
}

constexpr int kMaxSplit = kMaxBudget / kTPS;

// One workgroup per (sequence, head); thread d owns output dim d. The split
// weights e^{lse_s - max} are computed once into LDS, then every thread sums
// its column with independent loads.
__global__ __launch_bounds__(kDh) void merge_kernel(const float *__restrict__ part_o,
                                                    const float *__restrict__ part_lse, int n_split,
                                                    float *__restrict__ out)
{
    __shared__ float wgt[kMaxSplit];
    __shared__ float red[kDh / 64];
    const int bh = blockIdx.x;              // b * kHq + h
    const int tid = threadIdx.x;
    const float *lse = part_lse + (int64_t)bh * n_split;
    float ls = tid < n_split ? lse[tid] : -INFINITY;
    // block max of the split lse values (n_split <= 256 = threads)
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
#pragma unroll 8
        for (int s = 0; s < n_split; s++) {
            const float ws = wgt[s];
            const float x = col[(int64_t)s * kDh];   // empty splits hold stale data: select, not multiply
            den += ws;
            acc = ws != 0.0f ? fmaf(ws, x, acc) : acc;
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
                       static_cast<const uint8_t *>(kv), nullptr, 0, 0, nullptr, n_tok, nullptr, 0, 0, budget_tokens,
                       sm_scale, ws.part_o, ws.part_lse, ws.n_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_merge(ws, batch, out, s);
}

hipError_t launch_attention_paged(const uint16_t *q, const void *pool, const int32_t *pt, int64_t pt_stride,
                                  int64_t n_slots, const int32_t *sel, const int32_t *n_tok, const int32_t *ctx_len, int max_ctx,
                                  int batch, int budget_blocks, int budget_tokens, float sm_scale,
                                  const AttnWs &ws, float *out, hipStream_t s)
{
    dim3 grid((unsigned)ws.n_split, (unsigned)kHkv, (unsigned)batch);
    hipLaunchKernelGGL((attn_split_kernel<true>), grid, dim3(kThreads), 0, s, q,
                       static_cast<const uint8_t *>(pool), pt, pt_stride, n_slots, sel, n_tok, ctx_len, max_ctx,
                       budget_blocks, budget_tokens, sm_scale, ws.part_o, ws.part_lse, ws.n_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_merge(ws, batch, out, s);
}

} // namespace qsa
