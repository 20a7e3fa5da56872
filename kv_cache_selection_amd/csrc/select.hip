// select.hip -- budgeted C4-block selection.
//
// Keeps at most indexer_budget tokens per sequence (digest page, lead and
// mechanism sections) as whole C4 blocks (article intro): the forced blocks
// (sink at the start, the blocks of the tail ring at the end) plus the
// K - |F| best remaining blocks by (score desc, block index asc), returned in
// ascending block order. The result is exact -- the same set a full sort
// would give -- for any input, ties included.
//
// Radix selection over a monotone 32-bit key of the score:
//  1. (fused into scoring, or block_hist_kernel) a per-sequence histogram of
//     the key's top 12 bits over the non-forced blocks, built by many
//     workgroups with global atomics;
//  2. here, one workgroup per sequence finds the threshold bin b* from that
//     histogram and scans the sequence's block scores once, keeping the
//     blocks above b* ("definite") and the blocks inside b* ("candidates", as
//     64-bit composites key << 32 | ~index: unique, and ordered like
//     (score desc, index asc)) in LDS;
//  3. it picks the best need = K - |F| - |definite| candidates exactly -- by
//     rank counting when they fit in LDS, by a radix select over the
//     remaining 52 bits otherwise (candidates past the LDS capacity spill to
//     a global list only this workgroup touches) -- and writes the union in
//     ascending order through an LDS bitmap, so the output needs no sort.
// One workgroup owns a sequence from start to end, so no step needs a
// device-scope fence: on gfx950 such a fence writes back and invalidates the
// XCD's L2, which costs far more than this whole selection.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kPerThread = 64;                     // block scores per thread per pass (65536 per pass)
constexpr int kDefCap = kMaxBudget / kBT;          // definite blocks are < K <= 2048
constexpr int kCandCap = 2048;                     // candidates held in LDS
constexpr int kSegBlocks = 1 << 18;                // bitmap segment (32 KB of LDS)
constexpr int kSegWords = kSegBlocks / 32;
constexpr int kRadixBits = 13;
constexpr int kRadixBins = 1 << kRadixBits;        // 8192 bins = 32 KB
constexpr int kWorkWords = kSegWords > kRadixBins ? kSegWords : kRadixBins;

// LDS layout (dynamic): candidates | definite list | work area (histograms, bitmap)
constexpr size_t kSmemBytes = (size_t)kCandCap * 8 + (size_t)kDefCap * 4 + (size_t)kWorkWords * 4;

// Position of this lane's item in an LDS list: one LDS atomic per wave.
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t *counter)
{
    const uint64_t mask = __ballot(pred);
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

// Block-wide inclusive prefix sum of one uint32 per thread.
__device__ uint32_t block_inclusive_scan(uint32_t v, uint32_t *sh /* [16] */, uint32_t *total)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(v, d);
        if (lane >= d)
            v += o;
    }
    if (lane == 63)
        sh[wave] = v;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; w++) {
        const uint32_t x = sh[w];
        off += (w < wave) ? x : 0u;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return v + off;
}

// Walk a histogram of kThreads * W bins from the top: the bin where the
// running count first reaches `want`, and the count strictly above it.
template <int W>
__device__ void find_crossing(const uint32_t *h, uint32_t want, uint32_t *sh_scan, uint32_t *bin_out,
                              uint32_t *above_out)
{
    const int tr = kThreads - 1 - threadIdx.x;         // thread 0 owns the top bins
    uint32_t hv[W], local = 0;
#pragma unroll
    for (int i = 0; i < W; i++) {
        hv[i] = h[W * tr + i];
        local += hv[i];
    }
    uint32_t total;
    uint32_t above = block_inclusive_scan(local, sh_scan, &total) - local;
#pragma unroll
    for (int i = W - 1; i >= 0; i--) {
        if (above < want && above + hv[i] >= want) {
            *bin_out = W * tr + i;
            *above_out = above;
        }
        above += hv[i];
    }
    __syncthreads();
}

__global__ __launch_bounds__(kThreads) void select_kernel(
    const float *__restrict__ block_scores, int64_t bs_stride, const int32_t *__restrict__ ctx_len, int max_ctx,
    const uint32_t *__restrict__ hist, uint64_t *__restrict__ spill, int64_t spill_stride, int K, int sink_blocks,
    int tail_tokens, int32_t *__restrict__ sel, int32_t *__restrict__ n_sel, int32_t *__restrict__ n_tok)
{
    extern __shared__ uint64_t smem64[];
    uint64_t *cand = smem64;                                            // [kCandCap]
    int32_t *defl = reinterpret_cast<int32_t *>(smem64 + kCandCap);     // [kDefCap]
    uint32_t *work = reinterpret_cast<uint32_t *>(defl + kDefCap);      // [kWorkWords]
    __shared__ uint32_t sh_scan[16];
    __shared__ uint32_t sh_u[8];   // 0,1: crossing bin / count above; 2: #definite; 3: #candidates;
                                   // 4,5: T64; 6: partial last block taken

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = clamp_ctx(ctx_len[b], max_ctx);
    const int n = (L + kBT - 1) / kBT;
    int32_t *sel_b = sel + (int64_t)b * K;

    if (n <= K) {
        // Every block fits in the budget.
        for (int j = tid; j < K; j += kThreads)
            sel_b[j] = j < n ? j : -1;
        if (tid == 0) {
            n_sel[b] = n;
            if (n_tok)
                n_tok[b] = L;
        }
        return;
    }

    const int tail_first = tail_first_block(L, tail_tokens, n);
    const int r = K - forced_count(n, sink_blocks, tail_first);   // non-forced blocks to take (host: >= 0)

    const float *row = block_scores + (int64_t)b * bs_stride;
    uint64_t *spill_b = spill + (int64_t)b * spill_stride;
    // The first pass's scores are requested before anything waits on memory,
    // so their latency overlaps the histogram walk.
    float v[kPerThread];
    auto load_pass = [&](int base) {
#pragma unroll
        for (int k = 0; k < kPerThread; k++) {
            const int j = base + k * kThreads + tid;
            v[k] = j < n ? row[j] : 0.0f;
        }
    };
    if (r > 0)
        load_pass(0);

    // ---- 1. threshold bin b* from the 12-bit histogram ----------------------
    uint32_t bstar = kHistBins;   // no bin: nothing non-forced is taken
    if (tid == 0) {
        sh_u[0] = kHistBins;
        sh_u[1] = 0;
        sh_u[2] = 0;
        sh_u[3] = 0;
        sh_u[6] = 0;
    }
    __syncthreads();
    if (r > 0) {
        find_crossing<kHistBins / kThreads>(hist + (int64_t)b * kHistBins, (uint32_t)r, sh_scan, &sh_u[0],
                                            &sh_u[1]);
        bstar = sh_u[0];
    }

    // ---- 2. one pass over the block scores -----------------------------------
    if (r > 0) {
        for (int base = 0; base < n; base += kThreads * kPerThread) {
            if (base > 0)
                load_pass(base);
#pragma unroll
            for (int k = 0; k < kPerThread; k++) {
                const int j = base + k * kThreads + tid;
                bool is_def = false, is_cand = false;
                uint32_t key = 0;
                if (j < n && j >= sink_blocks && j < tail_first) {
                    key = order_key(v[k]);
                    const uint32_t bin = key >> kHistShift;
                    is_def = bin > bstar;
                    is_cand = bin == bstar;
                }
                const uint32_t pd = wave_append(is_def, &sh_u[2]);
                const uint32_t pc = wave_append(is_cand, &sh_u[3]);
                if (is_def && pd < (uint32_t)kDefCap)
                    defl[pd] = j;
                if (is_cand) {
                    const uint64_t comp = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
                    if (pc < (uint32_t)kCandCap)
                        cand[pc] = comp;
                    else if ((int64_t)pc < spill_stride)
                        spill_b[pc] = comp;
                }
            }
        }
    }
    __syncthreads();
    // The histogram describes these same scores, so D < r <= D + C; the clamps
    // only keep every index in bounds.
    const uint32_t D = r > 0 ? min(sh_u[2], (uint32_t)r) : 0u;
    const uint32_t C =
        r > 0 ? (uint32_t)min((int64_t)sh_u[3], spill_stride > kCandCap ? spill_stride : (int64_t)kCandCap) : 0u;
    const uint32_t need = min((uint32_t)r - D, C);

    // ---- 3a. threshold composite T64: chosen(i) <=> comp_i >= T64 -----------
    uint64_t T64 = ~0ull;
    if (need > 0 && need == C) {
        T64 = 0;
    } else if (need > 0 && C <= (uint32_t)kCandCap) {
        for (uint32_t i = tid; i < C; i += kThreads) {
            const uint64_t ci = cand[i];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < C; j++)
                rank += cand[j] > ci ? 1u : 0u;
            if (rank == need - 1) {     // the need-th largest composite
                sh_u[4] = (uint32_t)(ci >> 32);
                sh_u[5] = (uint32_t)ci;
            }
        }
        __syncthreads();
        T64 = ((uint64_t)sh_u[4] << 32) | sh_u[5];
    } else if (need > 0) {
        // Radix select over bits [51:0] in 4 passes of 13 bits (the top 12
        // bits are b* for every candidate).
        uint64_t prefix = (uint64_t)bstar << 52;
        uint64_t pmask = 0xFFFull << 52;
        uint32_t want = need;
        for (int shift = 52 - kRadixBits; shift >= 0; shift -= kRadixBits) {
            for (int i = tid; i < kRadixBins; i += kThreads)
                work[i] = 0;
            __syncthreads();
            for (uint32_t i = tid; i < C; i += kThreads) {
                const uint64_t c = i < (uint32_t)kCandCap ? cand[i] : spill_b[i];
                if ((c & pmask) == prefix)
                    atomicAdd(&work[(c >> shift) & (kRadixBins - 1)], 1u);
            }
            __syncthreads();
            find_crossing<kRadixBins / kThreads>(work, want, sh_scan, &sh_u[0], &sh_u[1]);
            const uint64_t digit = sh_u[0];
            want -= sh_u[1];
            prefix |= digit << shift;
            pmask |= (uint64_t)(kRadixBins - 1) << shift;
            __syncthreads();
        }
        T64 = prefix;
    }

    // ---- 3b. ascending output through a bitmap, segment by segment ----------
    uint32_t *bm = work;
    uint32_t written = 0;
    for (int seg0 = 0; seg0 < n; seg0 += kSegBlocks) {
        const int seg1 = min(seg0 + kSegBlocks, n);
        const int nw = (seg1 - seg0 + 31) / 32;
        __syncthreads();
        for (int i = tid; i < nw; i += kThreads)
            bm[i] = 0;
        __syncthreads();
        const int s_end = min(sink_blocks, n);
        for (int j = seg0 + tid; j < seg1; j += kThreads)
            if (j < s_end || j >= tail_first)
                atomicOr(&bm[(j - seg0) >> 5], 1u << ((j - seg0) & 31));
        for (uint32_t i = tid; i < D; i += kThreads) {
            const int j = defl[i];
            if (j >= seg0 && j < seg1)
                atomicOr(&bm[(j - seg0) >> 5], 1u << ((j - seg0) & 31));
        }
        if (need > 0) {
            for (uint32_t i = tid; i < C; i += kThreads) {
                const uint64_t c = i < (uint32_t)kCandCap ? cand[i] : spill_b[i];
                if (c >= T64) {
                    const int j = (int)(0xFFFFFFFFu - (uint32_t)c);
                    if (j >= seg0 && j < seg1)
                        atomicOr(&bm[(j - seg0) >> 5], 1u << ((j - seg0) & 31));
                }
            }
        }
        __syncthreads();
        if (tid == 0 && n - 1 >= seg0 && n - 1 < seg1)
            sh_u[6] = (bm[(n - 1 - seg0) >> 5] >> ((n - 1 - seg0) & 31)) & 1u;
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
    for (int p = (int)written + tid; p < K; p += kThreads)
        sel_b[p] = -1;
    if (tid == 0) {
        const int ns = (int)min(written, (uint32_t)K);
        n_sel[b] = ns;
        if (n_tok) {
            int nt = ns * kBT;
            const int last_len = L - (n - 1) * kBT;
            if (last_len < kBT && sh_u[6])
                nt -= kBT - last_len;     // the partial last block is selected
            n_tok[b] = nt;
        }
    }
}

} // namespace

hipError_t launch_select(const float *block_scores, int64_t bs_stride, const int32_t *ctx_len, int batch,
                         int max_ctx, const SelectWs &ws, int budget_blocks, int sink_blocks, int tail_tokens,
                         int32_t *sel, int32_t *n_sel, int32_t *n_tok, hipStream_t s)
{
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)batch), dim3(kThreads), kSmemBytes, s, block_scores, bs_stride,
                       ctx_len, max_ctx, ws.hist, ws.cand, ws.cand_stride, budget_blocks, sink_blocks, tail_tokens,
                       sel, n_sel, n_tok);
    return hipGetLastError();
}

} // namespace qsa
