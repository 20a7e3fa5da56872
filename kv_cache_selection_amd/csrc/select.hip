// select.hip -- budgeted C4-block selection.
//
// Keeps at most indexer_budget tokens per sequence (digest page, lead and
// mechanism sections) as whole C4 blocks (article intro): the forced blocks
// (sink at the start, the blocks of the tail ring at the end) plus the
// K - |F| best remaining blocks by (score desc, block index asc), returned in
// ascending block order. The result is exact -- the same set a full sort
// would give -- for any input, ties included.
//
// Radix selection over a monotone 32-bit key of the score, in three steps:
//  1. (fused into scoring, or block_hist_kernel) a per-sequence histogram of
//     the key's top 12 bits over the non-forced blocks;
//  2. every workgroup of a sequence finds the threshold bin b* from the
//     histogram, scans its slice of blocks and appends blocks above b*
//     ("definite") and blocks inside b* ("candidates", as 64-bit composites
//     key << 32 | ~index, unique and ordered like (score desc, index asc));
//  3. the last workgroup to finish (atomic ticket) picks the best
//     need = K - |F| - |definite| candidates exactly -- by rank counting in LDS
//     when there are few, by a radix select over the remaining 52 bits
//     otherwise -- and writes the union in ascending order through an LDS
//     bitmap, so the output needs no sort.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kSliceBlocks = 8192;          // blocks scanned per workgroup
constexpr int kRankMax = 2048;              // candidates ranked in LDS
constexpr int kSegBlocks = 1 << 18;         // bitmap segment (32 KB of LDS)
constexpr int kSegWords = kSegBlocks / 32;
constexpr int kRadixBits = 13;
constexpr int kRadixBins = 1 << kRadixBits; // 8192 bins = 32 KB

__device__ __forceinline__ uint32_t load_acquire(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_agent(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int32_t load_agent(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Position of this lane's item in a per-sequence list: one atomic per wave.
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t *counter)
{
    uint64_t mask = __ballot(pred);
    uint32_t base = 0;
    if (mask) {
        const int lane = threadIdx.x & 63;
        const int leader = __ffsll((unsigned long long)mask) - 1;
        if (lane == leader)
            base = atomicAdd(counter, (uint32_t)__popcll(mask));
        base = __shfl(base, leader);
        base += (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    }
    return base;
}

// Block-wide inclusive prefix sum of one uint32 per thread (kThreads = 1024).
__device__ uint32_t block_inclusive_scan(uint32_t v, uint32_t *sh /* [16] */, uint32_t *total)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t o = __shfl_up(v, d);
        if (lane >= d)
            v += o;
    }
    if (lane == 63)
        sh[wave] = v;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; w++) {
        uint32_t x = sh[w];
        off += (w < wave) ? x : 0u;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return v + off;
}

__global__ __launch_bounds__(kThreads) void select_kernel(
    const float *__restrict__ block_scores, int64_t bs_stride, const int32_t *__restrict__ ctx_len, int max_ctx,
    uint32_t *__restrict__ hist, uint32_t *__restrict__ counters, int32_t *__restrict__ def_list,
    uint64_t *__restrict__ cand, int64_t cand_stride, int K, int sink_blocks, int tail_tokens, int n_slices,
    int32_t *__restrict__ sel, int32_t *__restrict__ n_sel, int32_t *__restrict__ n_tok)
{
    extern __shared__ uint32_t smem[];       // max(kHistBins, kRadixBins, kSegWords) words + rank area
    __shared__ uint32_t sh_scan[16];
    __shared__ uint32_t sh_u[8];

    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int L = clamp_ctx(ctx_len[b], max_ctx);
    const int n = (L + kBT - 1) / kBT;
    int32_t *sel_b = sel + (int64_t)b * K;

    if (n <= K) {
        // Every block fits in the budget.
        if (blockIdx.x == 0) {
            for (int j = tid; j < K; j += kThreads)
                sel_b[j] = j < n ? j : -1;
            if (tid == 0) {
                n_sel[b] = n;
                if (n_tok)
                    n_tok[b] = L;
            }
        }
        return;
    }

    const int tail_first = tail_first_block(L, tail_tokens, n);
    const int n_forced = forced_count(n, sink_blocks, tail_first);
    const int r = K - n_forced;     // non-forced blocks to take (host guarantees >= 0)
    uint32_t *ctr = counters + (int64_t)b * kCounters;

    // ---- 1. threshold bin b* from the histogram ------------------------------
    // Thread t owns bins 4t..4t+3; walk from the top bin down.
    uint32_t bstar = kHistBins;   // "no bin": nothing non-forced is taken
    uint32_t above_bstar = 0;
    if (r > 0) {
        const uint32_t *gh = hist + (int64_t)b * kHistBins;
        const int tr = kThreads - 1 - tid;               // reversed thread order
        uint32_t h[4];
        uint32_t local = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            h[i] = gh[4 * tr + i];
            local += h[i];
        }
        uint32_t total;
        uint32_t incl = block_inclusive_scan(local, sh_scan, &total);   // over descending bin groups
        uint32_t above = incl - local;                   // count in bins > 4tr+3
        if (tid == 0)
            sh_u[0] = kHistBins;
        __syncthreads();
#pragma unroll
        for (int i = 3; i >= 0; i--) {
            if (above < (uint32_t)r && above + h[i] >= (uint32_t)r) {
                sh_u[0] = 4 * tr + i;
                sh_u[1] = above;
            }
            above += h[i];
        }
        __syncthreads();
        bstar = sh_u[0];
        above_bstar = sh_u[1];
    }

    // ---- 2. scan this slice ---------------------------------------------------
    const float *row = block_scores + (int64_t)b * bs_stride;
    const int j0 = blockIdx.x * kSliceBlocks;
    const int j1 = min(j0 + kSliceBlocks, n);
    if (r > 0) {
        for (int jb = j0; jb < j1; jb += kThreads) {
            const int j = jb + tid;
            bool is_def = false, is_cand = false;
            uint32_t key = 0;
            if (j < j1 && j >= sink_blocks && j < tail_first) {
                key = order_key(row[j]);
                const uint32_t bin = key >> kHistShift;
                is_def = bin > bstar;
                is_cand = bin == bstar;
            }
            uint32_t pd = wave_append(is_def, ctr + 0);
            uint32_t pc = wave_append(is_cand, ctr + 1);
            if (is_def && pd < (uint32_t)K)
                def_list[(int64_t)b * K + pd] = j;
            if (is_cand && pc < (uint64_t)cand_stride)
                cand[b * cand_stride + pc] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        }
    }

    // ---- ticket: the last workgroup of this sequence finishes ----------------
    __threadfence();
    __syncthreads();
    if (tid == 0)
        sh_u[2] = (atomicAdd(ctr + 2, 1u) == (uint32_t)(n_slices - 1)) ? 1u : 0u;
    __syncthreads();
    if (!sh_u[2])
        return;
    __threadfence();

    if (tid == 0)
        sh_u[7] = 0;
    // The histogram and the lists describe the same scores, so D < r <= D + C;
    // the clamps only keep every index in bounds.
    const uint32_t D = r > 0 ? min(load_acquire(ctr + 0), (uint32_t)r) : 0u;
    const uint32_t C = r > 0 ? (uint32_t)min((uint64_t)load_acquire(ctr + 1), (uint64_t)cand_stride) : 0u;
    const uint32_t need = min((uint32_t)r - D, C);  // candidates to take
    (void)above_bstar;
    const uint64_t *cb = cand + b * cand_stride;

    // ---- 3a. choose `need` candidates: threshold composite T64 -------------
    // chosen(i) <=> comp_i >= T64 (composites are unique).
    uint64_t T64 = ~0ull;
    if (need > 0 && need == C) {
        T64 = 0;
    } else if (need > 0 && C <= (uint32_t)kRankMax) {
        uint64_t *sc = reinterpret_cast<uint64_t *>(smem);
        for (uint32_t i = tid; i < C; i += kThreads)
            sc[i] = load_agent(cb + i);
        __syncthreads();
        if (tid == 0)
            sh_u[3] = 0, sh_u[4] = 0;
        __syncthreads();
        for (uint32_t i = tid; i < C; i += kThreads) {
            const uint64_t ci = sc[i];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < C; j++)
                rank += sc[j] > ci ? 1u : 0u;
            if (rank == need - 1) {     // the need-th largest composite
                sh_u[3] = (uint32_t)(ci >> 32);
                sh_u[4] = (uint32_t)ci;
            }
        }
        __syncthreads();
        T64 = ((uint64_t)sh_u[3] << 32) | sh_u[4];
    } else if (need > 0) {
        // Radix select over bits [51:0] in 4 passes of 13 bits (the top 12
        // bits are b* for every candidate).
        uint64_t prefix = (uint64_t)bstar << 52;
        uint64_t pmask = 0xFFFull << 52;
        uint32_t want = need;
        uint32_t *h = smem;
        for (int shift = 52 - kRadixBits; shift >= 0; shift -= kRadixBits) {
            for (int i = tid; i < kRadixBins; i += kThreads)
                h[i] = 0;
            __syncthreads();
            for (uint32_t i = tid; i < C; i += kThreads) {
                const uint64_t c = load_agent(cb + i);
                if ((c & pmask) == prefix)
                    atomicAdd(&h[(c >> shift) & (kRadixBins - 1)], 1u);
            }
            __syncthreads();
            // thread t owns bins [8t, 8t+8), walked from the top
            const int tr = kThreads - 1 - tid;
            uint32_t hv[8], local = 0;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                hv[i] = h[8 * tr + i];
                local += hv[i];
            }
            uint32_t total;
            uint32_t incl = block_inclusive_scan(local, sh_scan, &total);
            uint32_t above = incl - local;
#pragma unroll
            for (int i = 7; i >= 0; i--) {
                if (above < want && above + hv[i] >= want) {
                    sh_u[5] = 8 * tr + i;
                    sh_u[6] = above;
                }
                above += hv[i];
            }
            __syncthreads();
            const uint64_t digit = sh_u[5];
            want -= sh_u[6];
            prefix |= digit << shift;
            pmask |= (uint64_t)(kRadixBins - 1) << shift;
            __syncthreads();
        }
        T64 = prefix;
    }

    // ---- 3b. ascending output through a bitmap, segment by segment ----------
    uint32_t *bm = smem;
    uint32_t written = 0;
    for (int seg0 = 0; seg0 < n; seg0 += kSegBlocks) {
        const int seg1 = min(seg0 + kSegBlocks, n);
        const int nw = (seg1 - seg0 + 31) / 32;
        __syncthreads();
        for (int i = tid; i < nw; i += kThreads)
            bm[i] = 0;
        __syncthreads();
        // forced blocks
        const int s_end = min(sink_blocks, n);
        for (int j = seg0 + tid; j < seg1; j += kThreads) {
            if (j < s_end || j >= tail_first)
                atomicOr(&bm[(j - seg0) >> 5], 1u << ((j - seg0) & 31));
        }
        // definite blocks
        for (uint32_t i = tid; i < D; i += kThreads) {
            const int j = load_agent(def_list + (int64_t)b * K + i);
            if (j >= seg0 && j < seg1)
                atomicOr(&bm[(j - seg0) >> 5], 1u << ((j - seg0) & 31));
        }
        // chosen candidates
        if (need > 0) {
            for (uint32_t i = tid; i < C; i += kThreads) {
                const uint64_t c = load_agent(cb + i);
                if (c >= T64) {
                    const int j = (int)(0xFFFFFFFFu - (uint32_t)c);
                    if (j >= seg0 && j < seg1)
                        atomicOr(&bm[(j - seg0) >> 5], 1u << ((j - seg0) & 31));
                }
            }
        }
        __syncthreads();
        if (tid == 0 && n - 1 >= seg0 && n - 1 < seg1)
            sh_u[7] = (bm[(n - 1 - seg0) >> 5] >> ((n - 1 - seg0) & 31)) & 1u;
        // ordered compaction: thread t owns words [t*per, (t+1)*per)
        const int per = (nw + kThreads - 1) / kThreads;
        const int w0 = tid * per;
        const int w1 = min(w0 + per, nw);
        uint32_t cnt = 0;
        for (int i = w0; i < w1; i++)
            cnt += __popc(bm[i]);
        uint32_t total;
        uint32_t pos = written + block_inclusive_scan(cnt, sh_scan, &total) - cnt;
        for (int i = w0; i < w1; i++) {
            uint32_t m = bm[i];
            while (m) {
                const int bit = __ffs(m) - 1;
                m &= m - 1;
                if (pos < (uint32_t)K)
                    sel_b[pos] = seg0 + i * 32 + bit;
                pos++;
            }
        }
        written += total;
    }
    __syncthreads();
    for (int p = (int)written + tid; p < K; p += kThreads)
        sel_b[p] = -1;
    if (tid == 0) {
        const int ns = (int)min(written, (uint32_t)K);
        n_sel[b] = ns;
        if (n_tok) {
            // only the last block of the sequence can be partial
            int nt = ns * kBT;
            const int last_len = L - (n - 1) * kBT;
            if (last_len < kBT && sh_u[7])
                nt -= kBT - last_len;     // the partial last block is selected
            n_tok[b] = nt;
        }
    }
}

} // namespace

static size_t select_smem_bytes()
{
    size_t words = kHistBins;
    if ((size_t)kRadixBins > words)
        words = kRadixBins;
    if ((size_t)kSegWords > words)
        words = kSegWords;
    if ((size_t)kRankMax * 2 > words)
        words = (size_t)kRankMax * 2;
    return words * sizeof(uint32_t);
}

hipError_t launch_select(const float *block_scores, int64_t bs_stride, const int32_t *ctx_len, int batch,
                         int max_ctx, const SelectWs &ws, int budget_blocks, int sink_blocks, int tail_tokens,
                         int32_t *sel, int32_t *n_sel, int32_t *n_tok, hipStream_t s)
{
    const int n_blk_max = (max_ctx + kBT - 1) / kBT;
    const int n_slices = n_blk_max > 0 ? (n_blk_max + kSliceBlocks - 1) / kSliceBlocks : 1;
    dim3 grid((unsigned)n_slices, (unsigned)batch);
    hipLaunchKernelGGL(select_kernel, grid, dim3(kThreads), select_smem_bytes(), s, block_scores, bs_stride,
                       ctx_len, max_ctx, ws.hist, ws.counters, ws.def_list, ws.cand, ws.cand_stride, budget_blocks,
                       sink_blocks, tail_tokens, n_slices, sel, n_sel, n_tok);
    return hipGetLastError();
}

} // namespace qsa
