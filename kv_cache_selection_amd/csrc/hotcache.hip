// hotcache.hip -- a hot row cache in HBM in front of a KV pool in pinned host
// memory: only rows missing from the cache cross PCIe.
//
// The article's memory-ledger section keeps the full history in pinned host
// memory and only hot rows on the GPU, moving missing rows back on demand
// through a per-layer mapping of logical tokens to cache slots. Here each
// (layer, sequence) owns H cache rows (global ids b*H .. b*H + H - 1):
//   map[b][t]   = cache id holding logical token t, or -1;
//   owner[b][h] = logical token held by local row h, or -1.
// Per layer and step, after the selection:
//   1. hot_update_kernel (one workgroup per sequence): selected tokens already
//      cached are hits and keep their rows; the misses, in ascending token
//      order, take the rows no hit uses this step, in ascending row order,
//      unmapping each row's previous token. It writes the (token, row) fetch
//      list.
//   2. hot_fetch_kernel: copies each fetched token's row from the host pool
//      (through the page table) over PCIe into its cache row.
//   3. attention then reads every selected row from the cache, with `map` as
//      its page table (attention.hip, paged path).
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kUpdThreads = 1024;
constexpr int kMaxTokPerThread = kMaxBudget / kUpdThreads;   // 8
constexpr int kUsedWords = kMaxHot / 32;

__global__ __launch_bounds__(kUpdThreads) void hot_update_kernel(
    const int32_t *__restrict__ sel, const int32_t *__restrict__ n_tok, int budget_blocks, int budget_tokens,
    int max_ctx, int32_t *__restrict__ map, int64_t map_stride, int32_t *__restrict__ owner, int H,
    int2 *__restrict__ fetch, int32_t *__restrict__ n_fetch, int32_t *__restrict__ n_miss_out)
{
    __shared__ uint32_t used[kUsedWords];
    __shared__ int32_t miss_tok[kMaxBudget];
    __shared__ int32_t free_row[kMaxBudget];
    __shared__ uint32_t sh_scan[kUpdThreads / 64];

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    int nt = n_tok[b];
    nt = nt < 0 ? 0 : (nt > budget_tokens ? budget_tokens : nt);
    const int64_t base = (int64_t)b * H;
    int32_t *map_b = map + (int64_t)b * map_stride;
    int32_t *own_b = owner + base;

    for (int i = tid; i < (H + 31) / 32; i += kUpdThreads)
        used[i] = 0;
    __syncthreads();

    // Hits mark their rows; misses are compacted in ascending token order.
    int32_t tok[kMaxTokPerThread];
    bool miss[kMaxTokPerThread];
#pragma unroll
    for (int k = 0; k < kMaxTokPerThread; k++) {
        const int p = k * kUpdThreads + tid;
        tok[k] = -1;
        miss[k] = false;
        if (p < nt) {
            const int t = sel[(int64_t)b * budget_blocks + (p >> 2)] * kBT + (p & 3);
            if (t >= 0 && t < max_ctx) {
                tok[k] = t;
                const int64_t h = (int64_t)map_b[t] - base;
                if (h >= 0 && h < H)
                    atomicOr(&used[h >> 5], 1u << (h & 31));
                else
                    miss[k] = true;
            }
        }
    }
    uint32_t n_miss = 0;
#pragma unroll
    for (int k = 0; k < kMaxTokPerThread; k++) {
        if (k * kUpdThreads >= nt)
            break;                                  // uniform
        uint32_t tot;
        const uint32_t pos = n_miss + block_inclusive_scan<kUpdThreads>(miss[k] ? 1u : 0u, sh_scan, &tot) - 1u;
        if (miss[k])
            miss_tok[pos] = tok[k];
        n_miss += tot;
    }
    __syncthreads();                                // `used` is complete

    // Rows no hit uses, in ascending order: thread i owns bitmap word i
    // (and i + kUpdThreads, ... for larger caches).
    uint32_t n_free = 0;
    for (int w0 = 0; w0 < (H + 31) / 32; w0 += kUpdThreads) {
        const int w = w0 + tid;
        uint32_t avail = 0;
        if (w < (H + 31) / 32) {
            avail = ~used[w];
            if (w == (H - 1) / 32 && (H & 31))
                avail &= (1u << (H & 31)) - 1u;     // rows beyond H
        }
        const uint32_t cnt = __popc(avail);
        uint32_t tot;
        uint32_t pos = n_free + block_inclusive_scan<kUpdThreads>(cnt, sh_scan, &tot) - cnt;
        while (avail && pos < n_miss) {
            const int bit = __ffs(avail) - 1;
            avail &= avail - 1;
            free_row[pos++] = w * 32 + bit;
        }
        n_free += tot;
        if (n_free >= n_miss)
            break;                                  // uniform
    }
    __syncthreads();

    // Misses take the free rows; each row's previous token loses its mapping.
    // Host-side checks guarantee H >= budget, hence n_free >= n_miss.
    const uint32_t n_take = n_miss < n_free ? n_miss : n_free;
    for (uint32_t i = tid; i < n_take; i += kUpdThreads) {
        const int t = miss_tok[i];
        const int h = free_row[i];
        const int old = own_b[h];
        if (old >= 0 && old < max_ctx)
            map_b[old] = -1;
        own_b[h] = t;
        map_b[t] = (int32_t)(base + h);
        fetch[(int64_t)b * budget_tokens + i] = make_int2(t, h);
    }
    if (tid == 0) {
        n_fetch[b] = (int32_t)n_take;
        if (n_miss_out)
            n_miss_out[b] = (int32_t)n_take;
    }
}

// Copy the fetched rows, host pool -> cache: 16 fetches per workgroup, 16
// bytes per lane and piece so that each row is one contiguous 2 KB read.
constexpr int kFetchThreads = 256;
constexpr int kFetchPerWg = 16;
constexpr int kPieces = kRowBytes / 16;

__global__ __launch_bounds__(kFetchThreads) void hot_fetch_kernel(
    const int2 *__restrict__ fetch, const int32_t *__restrict__ n_fetch, int budget_tokens,
    const int32_t *__restrict__ pt, int64_t pt_stride, int64_t n_slots, int max_ctx, const u32x4 *__restrict__ pool,
    u32x4 *__restrict__ rows, int H, uint32_t *flags)
{
    const int b = blockIdx.y;
    int nf = n_fetch[b];
    nf = nf < 0 ? 0 : (nf > budget_tokens ? budget_tokens : nf);
    const int i0 = blockIdx.x * kFetchPerWg;
    if (i0 >= nf)
        return;
    constexpr int kPer = kFetchPerWg * kPieces / kFetchThreads;   // 8 pieces per thread
    u32x4 v[kPer];
    int64_t dst[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int c = threadIdx.x + k * kFetchThreads;
        const int i = i0 + c / kPieces;
        const int piece = c % kPieces;
        dst[k] = -1;
        if (i < nf) {
            const int2 f = fetch[(int64_t)b * budget_tokens + i];
            if (f.x >= 0 && f.x < max_ctx && f.y >= 0 && f.y < H) {
                const int32_t raw = pt[(int64_t)b * pt_stride + f.x];
                const int64_t slot = safe_slot(raw, n_slots);
                if (piece == 0 && slot != raw)
                    raise_flag(flags, QSA_FLAG_BAD_SLOT);
                v[k] = __builtin_nontemporal_load(pool + slot * kPieces + piece);
                dst[k] = ((int64_t)b * H + f.y) * kPieces + piece;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kPer; k++)
        if (dst[k] >= 0)
            rows[dst[k]] = v[k];
}

__global__ void fill_i32_kernel(int32_t *__restrict__ p, int64_t n, int32_t v)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = v;
}

} // namespace

hipError_t launch_hot_update(const int32_t *sel, const int32_t *n_tok, int batch, int budget_blocks,
                             int budget_tokens, int max_ctx, int32_t *map, int64_t map_stride, int32_t *owner, int H,
                             int2 *fetch, int32_t *n_fetch, int32_t *n_miss_out, hipStream_t s)
{
    hipLaunchKernelGGL(hot_update_kernel, dim3((unsigned)batch), dim3(kUpdThreads), 0, s, sel, n_tok, budget_blocks,
                       budget_tokens, max_ctx, map, map_stride, owner, H, fetch, n_fetch, n_miss_out);
    return hipGetLastError();
}

hipError_t launch_hot_fetch(const int2 *fetch, const int32_t *n_fetch, int batch, int budget_tokens,
                            const int32_t *pt, int64_t pt_stride, int64_t n_slots, int max_ctx, const void *pool,
                            void *rows, int H, uint32_t *flags, hipStream_t s)
{
    dim3 grid((unsigned)((budget_tokens + kFetchPerWg - 1) / kFetchPerWg), (unsigned)batch);
    hipLaunchKernelGGL(hot_fetch_kernel, grid, dim3(kFetchThreads), 0, s, fetch, n_fetch, budget_tokens, pt,
                       pt_stride, n_slots, max_ctx, static_cast<const u32x4 *>(pool), static_cast<u32x4 *>(rows), H,
                       flags);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

} // namespace qsa
