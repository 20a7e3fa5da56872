// index_score.hip -- indexer scoring and C4 block reduce.
//
// For every cached token t of sequence b (digest page, mechanism section: the
// GPU-resident index of 66-byte keys is scanned every decode step):
//     s_t = sum_h w_h * ReLU(sigma_t * (q_h . k_t))
// and for every C4 block j (article intro: 4 adjacent tokens form the unit
// of selection) B_j = max of s_t over the block's valid tokens.
//
// Mapping on gfx950: a wave scores a tile of 64 tokens on the matrix cores,
// one token per lane (idx_tile_load / idx_tile_score, shared with the
// selection kernel, which scores a chunk again when it must). The VALU only
// widens codes and runs the ReLU/weight epilogue and the block max, so the
// kernel stays bound by HBM, not by fp32 FMA throughput.
//
// One launch may scan several layers (grid z), their pointers in the kernel
// arguments, so that the scan streams from one layer into the next.
//
// For the long-context selection (sequences with more blocks than the budget
// and than the one-workgroup selection holds), each workgroup also builds an
// LDS histogram of the top 12 bits of its blocks' order keys (forced blocks
// excluded) and from it the chunk's candidate list: its best blocks, cut at a
// bin boundary (build_chunk_list). The selection then starts from these
// lists, so nothing needs to be counted across workgroups, and no global
// histogram has to be cleared before the scan. In the decode step
// (drop_listed_bs) such a chunk stores its block scores only when its list
// was cut short by a crowded bin: the 24 MB of block scores of a 12-layer
// batch8-256k step took about 18 us of its scan (266 against 249 us), and the
// selection reads a chunk's scores back only in the rare case that it must
// re-read the chunk, scoring it again from the index otherwise.
#include "qsa_internal.h"

#include <hip/hip_ext.h>

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kThreads = 512;                      // 8 waves: half as many histogram clears
constexpr int kWaveTok = 64;                       // tokens per wave iteration
constexpr int kWgTok = kThreads / 64 * kWaveTok;   // 512 tokens per workgroup iteration
constexpr int kMaxChunkTokens = kMaxScoreChunkTokens;
static_assert(kWgTok == kScoreWgTokens, "chunks are whole workgroup iterations");

// Grid (chunks of chunk_tokens, B, layers).
template <bool kTokens, bool kLists, int N>
__global__ __launch_bounds__(kThreads) void index_score_kernel(const ScoreLayersT<N> Ls,
                                                               const int32_t *__restrict__ ctx_len,
                                                               const int64_t *__restrict__ row0, int64_t n_rows,
                                                               int max_ctx, int chunk_tokens, int64_t bs_stride,
                                                               ListGeom g, int budget_blocks, int sink_blocks,
                                                               int tail_tokens, uint32_t *clear_flags)
{
    __shared__ uint32_t lhist[kLists ? kHistBins : 1];
    __shared__ uint32_t lsh[5];                    // highest key bin; list threshold, fill, size and keep
    // The chunk's block scores, written out at the end as contiguous rows
    // with non-temporal stores. Their 2 MB per layer are 1.5 % of the bytes,
    // but stored from the loop with ordinary stores they slowed the 12-layer
    // scan by about 30 µs; written this way they cost about half that.
    __shared__ float lbs[kMaxChunkTokens / kBT];
    const uint8_t *__restrict__ keys = Ls.keys[blockIdx.z];
    const uint16_t *__restrict__ scales = Ls.scales[blockIdx.z];
    float *__restrict__ token_scores = Ls.token_scores[blockIdx.z];
    float *__restrict__ block_scores = Ls.block_scores[blockIdx.z];

    // The call's flags word is cleared here, before anything of the call can
    // raise a flag: this launch raises none (the selection reports what it
    // would), and every later kernel of the call follows it on its stream.
    if (clear_flags && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)
        *clear_flags = 0u;

    const int b = blockIdx.y;
    const int64_t r0 = row0[b];
    const int32_t L_raw = ctx_len[b];
    int L = clamp_ctx(L_raw, max_ctx);
    const bool bad_rows = r0 < 0 || r0 + L > n_rows;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (L != L_raw)
            raise_flag(Ls.flags, QSA_FLAG_BAD_CTX_LEN);
        if (bad_rows && L > 0)
            raise_flag(Ls.flags, QSA_FLAG_BAD_INDEX_ROWS);
    }
    if (bad_rows)
        L = 0;                                    // rows outside the index buffer: empty
    const int t_begin = blockIdx.x * chunk_tokens;
    if (t_begin >= L)
        return;
    const int n_blk = (L + kBT - 1) / kBT;
    const bool do_hist = kLists && n_blk > budget_blocks;
    const int tail_first = tail_first_block(L, tail_tokens, n_blk);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint8_t *kbase = keys + r0 * kIdxD;
    const uint16_t *sbase = scales + r0;
    float *bs_row = block_scores + (int64_t)b * bs_stride;
    const int t_end = min(t_begin + chunk_tokens, L);
    const int blk_begin = t_begin / kBT;

    // Two-deep software pipeline: the keys of the wave's next 64 tokens are
    // requested before the current 64 are widened and multiplied. The first
    // tile is requested before anything else is set up.
    idx_u32x4 k[4], kn[4];
    uint16_t sc_bits = 0, sc_next = 0;
    int tw = t_begin + wave * kWaveTok;
    if (tw < t_end)
        idx_tile_load(kbase, sbase, tw, L, lane, k, sc_bits);

    if (do_hist) {
        for (int i = tid; i < kHistBins; i += kThreads)
            lhist[i] = 0;
        if (tid == 0)
            lsh[0] = 0;
    }
    uint32_t top = 0;                       // highest key bin of this lane's eligible blocks
    IdxQuery Q;
    idx_query(Ls.q_idx[blockIdx.z] + (int64_t)b * kIdxH * kIdxD, Ls.w_idx[blockIdx.z] + (int64_t)b * kIdxH, lane, Q);

    if (do_hist)
        __syncthreads();

    for (; tw < t_end; tw += kWgTok) {
        const int tn = tw + kWgTok;
        if (tn < t_end)
            idx_tile_load(kbase, sbase, tn, L, lane, kn, sc_next);
        const int t = tw + lane;
        const bool valid = t < L;
        float s = idx_tile_score(k, sc_bits, Q);
        if (!valid)
            s = -INFINITY;
        if (kTokens && valid)
            token_scores[r0 + t] = s;

        // C4 block = 4 consecutive lanes (t is a multiple of 64 at lane 0).
        s = fmaxf(s, __shfl_xor(s, 1));
        s = fmaxf(s, __shfl_xor(s, 2));
        const int blk = t >> 2;
        if ((lane & 3) == 0 && blk < n_blk) {
            lbs[blk - blk_begin] = s;
            if (do_hist && blk >= sink_blocks && blk < tail_first) {
                const uint32_t bin = order_key(s) >> kHistShift;
                atomicAdd(&lhist[bin], 1u);
                top = bin > top ? bin : top;
            }
        }
#pragma unroll
        for (int g = 0; g < 4; g++)
            k[g] = kn[g];
        sc_bits = sc_next;
    }

    if (do_hist) {
        top = wave_max(top);
        if (lane == 0)
            atomicMax(&lsh[0], top);
    }
    __syncthreads();
    const int blk_end = min(blk_begin + chunk_tokens / kBT, n_blk);
    bool store = true;
    if (do_hist) {
        const int64_t c = (int64_t)b * g.n_chunks + blockIdx.x;
        store = build_chunk_list<kThreads>(lhist, lbs, blk_begin, blk_end, sink_blocks, tail_first, g.m, g.cap,
                                           (int)lsh[0], !Ls.drop_listed_bs, lsh + 1, Ls.heads[blockIdx.z] + c,
                                           Ls.lists[blockIdx.z] + c * g.cap);
    }
    if (store)
        for (int j = blk_begin + tid; j < blk_end; j += kThreads)
            __builtin_nontemporal_store(lbs[j - blk_begin], bs_row + j);
}

// Chunk lists of existing block scores (standalone selection call): the
// same lists the scan builds, one workgroup per chunk. Grid (n_chunks, B).
__global__ __launch_bounds__(kThreads) void list_build_kernel(const float *__restrict__ block_scores,
                                                              int64_t bs_stride, const int32_t *__restrict__ ctx_len,
                                                              int max_ctx, ListGeom g, uint32_t *__restrict__ heads,
                                                              uint64_t *__restrict__ lists, int budget_blocks,
                                                              int sink_blocks, int tail_tokens)
{
    __shared__ uint32_t lhist[kHistBins];
    __shared__ float lbs[kMaxChunkTokens / kBT];
    __shared__ uint32_t lsh[5];
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int L = clamp_ctx(ctx_len[b], max_ctx);
    const int n_blk = (L + kBT - 1) / kBT;
    const int j0 = blockIdx.x * g.chunk_blocks;
    if (n_blk <= budget_blocks || j0 >= n_blk)
        return;
    const int tail_first = tail_first_block(L, tail_tokens, n_blk);
    const int j1 = min(j0 + g.chunk_blocks, n_blk);
    for (int i = tid; i < kHistBins; i += kThreads)
        lhist[i] = 0;
    if (tid == 0)
        lsh[0] = 0;
    __syncthreads();
    const float *row = block_scores + (int64_t)b * bs_stride;
    uint32_t top = 0;
    for (int j = j0 + tid; j < j1; j += kThreads) {
        const float v = row[j];
        lbs[j - j0] = v;
        if (j >= sink_blocks && j < tail_first) {
            const uint32_t bin = order_key(v) >> kHistShift;
            atomicAdd(&lhist[bin], 1u);
            top = bin > top ? bin : top;
        }
    }
    top = wave_max(top);
    if ((tid & 63) == 0)
        atomicMax(&lsh[0], top);
    __syncthreads();
    const int64_t c = (int64_t)b * g.n_chunks + blockIdx.x;
    (void)build_chunk_list<kThreads>(lhist, lbs, j0, j1, sink_blocks, tail_first, g.m, g.cap, (int)lsh[0], true,
                                     lsh + 1, heads + c, lists + c * g.cap);
}

__global__ void zero_u32_kernel(uint32_t *__restrict__ p, int64_t n)
{
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = 0;
}

__global__ void copy_u32_kernel(const uint32_t *__restrict__ src, uint32_t *__restrict__ dst, int64_t n)
{
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

} // namespace

hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 2048)
        blocks = 2048;
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_copy_u32(const uint32_t *src, uint32_t *dst, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 2048)
        blocks = 2048;
    hipLaunchKernelGGL(copy_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

// With a start/stop event pair the launch goes through hipExtLaunchKernel,
// whose events take the kernel's own begin and end timestamps.
template <typename Kernel, typename... Args>
void launch_timed(Kernel k, dim3 grid, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, Args... args)
{
    if (ev0 && ev1)
        hipExtLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, ev0, ev1, 0, args...);
    else
        hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, args...);
}

template <int N>
static hipError_t launch_score_n(const ScoreLayersT<N> &L, int n_layers, const int32_t *ctx_len,
                                 const int64_t *row0, int64_t n_rows, int batch, int max_ctx, int64_t bs_stride,
                                 const ListGeom &g, int budget_blocks, int sink_blocks, int tail_tokens,
                                 hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, uint32_t *clear_flags)
{
    const int chunk = score_chunk_tokens(batch, max_ctx);
    const int n_chunks = (max_ctx + chunk - 1) / chunk;
    if (L.heads[0] && (g.chunk_blocks * kBT != chunk || g.n_chunks != n_chunks || n_chunks > kMaxListChunks ||
                       g.m < 1 || g.m > g.cap || g.cap > kListCap || g.cap > kThreads))
        return hipErrorInvalidValue;
    dim3 grid((unsigned)n_chunks, (unsigned)batch, (unsigned)n_layers);
#define QSA_SCORE_ARGS \
    L, ctx_len, row0, n_rows, max_ctx, chunk, bs_stride, g, budget_blocks, sink_blocks, tail_tokens, clear_flags
    if (L.token_scores[0]) {
        if (L.heads[0])
            launch_timed(index_score_kernel<true, true, N>, grid, s, ev0, ev1, QSA_SCORE_ARGS);
        else
            launch_timed(index_score_kernel<true, false, N>, grid, s, ev0, ev1, QSA_SCORE_ARGS);
    } else {
        if (L.heads[0])
            launch_timed(index_score_kernel<false, true, N>, grid, s, ev0, ev1, QSA_SCORE_ARGS);
        else
            launch_timed(index_score_kernel<false, false, N>, grid, s, ev0, ev1, QSA_SCORE_ARGS);
    }
#undef QSA_SCORE_ARGS
    return hipGetLastError();
}

hipError_t launch_index_score_layers(const ScoreLayers &L, int n_layers, const int32_t *ctx_len, const int64_t *row0,
                                     int64_t n_rows, int batch, int max_ctx, int64_t bs_stride, const ListGeom &g,
                                     int budget_blocks, int sink_blocks, int tail_tokens, hipStream_t s,
                                     hipEvent_t ev0, hipEvent_t ev1, uint32_t *clear_flags)
{
    if (n_layers < 1 || n_layers > kMaxChainLayers || (clear_flags && L.flags))
        return hipErrorInvalidValue;
    if (max_ctx <= 0) {
        // nothing to scan: the flags word is still cleared for the call
        if (clear_flags)
            return launch_zero_u32(clear_flags, 1, s);
        return hipSuccess;
    }
    for (int l = 1; l < n_layers; l++)
        if (!L.token_scores[l] != !L.token_scores[0] || !L.heads[l] != !L.heads[0] ||
            (L.heads[l] && !L.lists[l]))
            return hipErrorInvalidValue;
    if (L.heads[0] && !L.lists[0])
        return hipErrorInvalidValue;
    if (n_layers > 1)
        return launch_score_n(L, n_layers, ctx_len, row0, n_rows, batch, max_ctx, bs_stride, g, budget_blocks,
                              sink_blocks, tail_tokens, s, ev0, ev1, clear_flags);
    const ScoreLayersT<1> L1 = {{L.keys[0]},         {L.scales[0]},       {L.q_idx[0]}, {L.w_idx[0]},
                                {L.token_scores[0]}, {L.block_scores[0]}, {L.heads[0]}, {L.lists[0]},
                                L.flags,             L.drop_listed_bs};
    return launch_score_n(L1, 1, ctx_len, row0, n_rows, batch, max_ctx, bs_stride, g, budget_blocks, sink_blocks,
                          tail_tokens, s, ev0, ev1, clear_flags);
}

hipError_t launch_index_score(const uint8_t *keys, const uint16_t *scales, const uint16_t *q_idx,
                              const float *w_idx, const int32_t *ctx_len, const int64_t *row0, int64_t n_rows,
                              int batch, int max_ctx, float *token_scores, float *block_scores, int64_t bs_stride,
                              uint32_t *heads, uint64_t *lists, const ListGeom &g, int budget_blocks,
                              int sink_blocks, int tail_tokens, uint32_t *flags, hipStream_t s, hipEvent_t ev0,
                              hipEvent_t ev1, uint32_t *clear_flags, bool drop_listed_bs)
{
    ScoreLayers L = {};
    L.flags = flags;
    L.drop_listed_bs = drop_listed_bs ? 1 : 0;
    L.keys[0] = keys;
    L.scales[0] = scales;
    L.q_idx[0] = q_idx;
    L.w_idx[0] = w_idx;
    L.token_scores[0] = token_scores;
    L.block_scores[0] = block_scores;
    L.heads[0] = heads;
    L.lists[0] = lists;
    return launch_index_score_layers(L, 1, ctx_len, row0, n_rows, batch, max_ctx, bs_stride, g, budget_blocks,
                                     sink_blocks, tail_tokens, s, ev0, ev1, clear_flags);
}

hipError_t launch_list_build(const float *block_scores, int64_t bs_stride, const int32_t *ctx_len, int batch,
                             int max_ctx, uint32_t *heads, uint64_t *lists, const ListGeom &g, int budget_blocks,
                             int sink_blocks, int tail_tokens, hipStream_t s)
{
    const int n_blk_max = (max_ctx + kBT - 1) / kBT;
    if (n_blk_max <= 0)
        return hipSuccess;
    if (g.chunk_blocks < 1 || g.chunk_blocks > kMaxChunkTokens / kBT || g.n_chunks > kMaxListChunks ||
        (int64_t)g.n_chunks * g.chunk_blocks < n_blk_max || g.m < 1 || g.m > g.cap || g.cap > kListCap ||
        g.cap > kThreads)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)g.n_chunks, (unsigned)batch);
    hipLaunchKernelGGL(list_build_kernel, grid, dim3(kThreads), 0, s, block_scores, bs_stride, ctx_len, max_ctx, g,
                       heads, lists, budget_blocks, sink_blocks, tail_tokens);
    return hipGetLastError();
}

} // namespace qsa
