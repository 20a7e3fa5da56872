// select.hip -- budgeted C4-block selection.
//
// Keeps at most indexer_budget tokens per sequence (digest page, lead and
// mechanism sections) as whole C4 blocks (article intro): the forced blocks
// (sink at the start, the blocks of the tail ring at the end) plus the
// K - |F| best remaining blocks by (score desc, block index asc), returned in
// ascending block order. The result is exact -- the same set a full sort
// would give -- for any input, ties included.
//
// Radix selection over a monotone 32-bit key of the score, in three kernels:
//  1. (fused into scoring, or block_hist_kernel) a per-sequence histogram of
//     the key's top 12 bits over the non-forced blocks;
//  2. collect_kernel: one workgroup per slice of 2048 blocks finds the
//     threshold bin b* from the histogram and writes the slice's blocks
//     above b* ("definite") and inside b* ("candidates", as 64-bit
//     composites key << 32 | ~index: unique, and ordered like (score desc,
//     index asc)) with their counts to the slice's own slot;
//  3. finish_kernel: one workgroup per sequence gathers the slots through
//     prefix offsets, picks the best need = K - |F| - |definite| candidates
//     exactly with a radix select over the composites' remaining 64 - 12 bits
//     (11-bit digits, finishing by direct ranking once few are left), and
//     writes the union in ascending order through an LDS bitmap, so the
//     output needs no sort.
// Sequences of up to 16,384 blocks (65,536 tokens) skip steps 2 and 3:
// select_one_kernel holds all of a sequence's scores in one workgroup's
// registers and selects in one launch (radix passes over the registers, and
// an equal-key bitmap for the ties of the last key).
// Nothing is shared between workgroups inside a kernel: no global atomics on
// a few hot addresses (they serialise at the memory side) and no
// device-scope fences (on gfx950 one writes back and invalidates the XCD's
// L2). The kernel boundary orders the slots, and the scan of the scores is
// spread over many CUs. One launch may cover several layers (grid z for
// collect_kernel, y for finish_kernel): their pointers travel in the kernel
// arguments.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 1024;                     // finish_kernel
constexpr int kCollectThreads = 256;
constexpr int kCollectPer = 8;                     // block scores per thread in collect_kernel
constexpr int kCandCap = 2048;                     // candidates held in LDS by finish_kernel
constexpr int kSegBlocks = 1 << 18;                // bitmap segment (32 KB of LDS)
constexpr int kSegWords = kSegBlocks / 32;
constexpr int kDigitBits = 11;                     // radix digit of the candidate selection
constexpr int kDigitBins = 1 << kDigitBits;        // 2048 bins, 2 per thread
constexpr int kWorkWords = kSegWords;              // bitmap; also digit histogram + short list
constexpr int kDefCap = kMaxBudget / kBT;          // definite blocks are < K <= 2048
constexpr int kMaxSlices = (kMaxCtx / kBT) / kSliceBlocks;   // 256
static_assert(kSliceBlocks == kCollectThreads * kCollectPer, "slice size");
static_assert(kMaxSlices <= kThreads, "one finish thread per slice");
static_assert(kDigitBins + 2 * kThreads <= kWorkWords, "digit histogram and short list fit the work area");

// finish_kernel LDS layout (dynamic): candidates | definite list | work area
// (digit histogram and short list, then the output bitmap)
constexpr size_t kSmemBytes = (size_t)kCandCap * 8 + (size_t)kDefCap * 4 + (size_t)kWorkWords * 4;

// Walk a histogram of NT * W bins from the top: the bin where the running
// count first reaches `want`, and the count strictly above it. Thread i
// holds bins W (NT - 1 - i) .. + W - 1 in hv, so thread 0 holds the top ones.
template <int W, int NT>
__device__ void crossing_of(const uint32_t (&hv)[W], uint32_t want, uint32_t *sh_scan, uint32_t *bin_out,
                            uint32_t *above_out, uint32_t *in_bin_out = nullptr)
{
    const int tr = NT - 1 - threadIdx.x;
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < W; i++)
        local += hv[i];
    uint32_t total;
    uint32_t above = block_inclusive_scan<NT>(local, sh_scan, &total) - local;
#pragma unroll
    for (int i = W - 1; i >= 0; i--) {
        if (above < want && above + hv[i] >= want) {
            *bin_out = W * tr + i;
            *above_out = above;
            if (in_bin_out)
                *in_bin_out = hv[i];
        }
        above += hv[i];
    }
    __syncthreads();
}

// The same over a histogram in memory.
template <int W, int NT>
__device__ void find_crossing(const uint32_t *h, uint32_t want, uint32_t *sh_scan, uint32_t *bin_out,
                              uint32_t *above_out)
{
    const int tr = NT - 1 - threadIdx.x;
    uint32_t hv[W];
#pragma unroll
    for (int i = 0; i < W; i++)
        hv[i] = h[W * tr + i];
    crossing_of<W, NT>(hv, want, sh_scan, bin_out, above_out);
}

// Number of non-forced blocks to take, or -1 when every block fits.
__device__ __forceinline__ int rest_to_take(int L, int n, int K, int sink_blocks, int tail_tokens, int *tail_first)
{
    if (n <= K)
        return -1;
    *tail_first = tail_first_block(L, tail_tokens, n);
    return K - forced_count(n, sink_blocks, *tail_first);   // host guarantees >= 0
}

// Grid (n_slices, B, layers).
template <int N>
__global__ __launch_bounds__(kCollectThreads) void collect_kernel(const SelectLayersT<N> Ls, int64_t bs_stride,
                                                                  const int32_t *__restrict__ ctx_len, int max_ctx,
                                                                  int n_slices, int K, int sink_blocks,
                                                                  int tail_tokens)
{
    const float *__restrict__ block_scores = Ls.bs[blockIdx.z];
    const uint32_t *__restrict__ hist = Ls.ws[blockIdx.z].hist;
    uint32_t *__restrict__ slot_count = Ls.ws[blockIdx.z].slot_count;
    int32_t *__restrict__ slot_def = Ls.ws[blockIdx.z].slot_def;
    uint64_t *__restrict__ slot_cand = Ls.ws[blockIdx.z].slot_cand;
    __shared__ uint32_t sh_scan[kCollectThreads / 64];
    __shared__ uint32_t sh_u[4];                    // 0,1: crossing bin / count above; 2,3: list lengths

    const int b = blockIdx.y;
    const int slice = blockIdx.x;
    const int tid = threadIdx.x;
    const SelectWs &ws = Ls.ws[blockIdx.z];
    const int L = select_len(ctx_len[b], ws.row0 ? ws.row0[b] : 0, max_ctx, ws);
    const int n = (L + kBT - 1) / kBT;
    const int j0 = slice * kSliceBlocks;
    int tail_first = n;
    const int r = rest_to_take(L, n, K, sink_blocks, tail_tokens, &tail_first);
    if (r <= 0 || j0 >= n)
        return;

    // The histogram copies of the sequence are requested first, then the
    // slice's scores, whose latency overlaps the histogram walk. The score
    // reads are unconditional (past the end they repeat the last block,
    // whose copies are never used): the compiler can then count them, and
    // since loads are counted in the order they were issued, the walk waits
    // only for the histogram.
    constexpr int W = kHistBins / kCollectThreads;
    const uint32_t *hb = hist + ((int64_t)b * kHistReps * kHistBins + W * (kCollectThreads - 1 - tid));
    uint32_t hraw[kHistReps][W];
#pragma unroll
    for (int c = 0; c < kHistReps; c++)
#pragma unroll
        for (int i = 0; i < W; i++)
            hraw[c][i] = hb[c * kHistBins + i];
    const float *row = block_scores + (int64_t)b * bs_stride;
    float v[kCollectPer];
#pragma unroll
    for (int k = 0; k < kCollectPer; k++)
        v[k] = row[min(j0 + k * kCollectThreads + tid, n - 1)];
    uint32_t hv[W];
#pragma unroll
    for (int i = 0; i < W; i++) {
        hv[i] = 0;
#pragma unroll
        for (int c = 0; c < kHistReps; c++)
            hv[i] += hraw[c][i];
    }
    if (tid == 0) {
        sh_u[0] = kHistBins;
        sh_u[2] = 0;
        sh_u[3] = 0;
    }
    __syncthreads();
    crossing_of<W, kCollectThreads>(hv, (uint32_t)r, sh_scan, &sh_u[0], &sh_u[1]);
    const uint32_t bstar = sh_u[0];

    // The slot is this workgroup's own: list entries go straight to it. A
    // wave ballots its items first, takes room for all of them with one LDS
    // atomic per list, and places each item by the popcounts of the ballots.
    const int64_t slot = (int64_t)b * n_slices + slice;
    int32_t *my_def = slot_def + slot * kSliceBlocks;
    uint64_t *my_cand = slot_cand + slot * kSliceBlocks;
    const int lane = tid & 63;
    const uint64_t lt = (1ull << lane) - 1ull;
    uint64_t md[kCollectPer], mc[kCollectPer];
    uint32_t key[kCollectPer];
    uint32_t nd = 0, nc = 0;
#pragma unroll
    for (int k = 0; k < kCollectPer; k++) {
        const int j = j0 + k * kCollectThreads + tid;
        bool is_def = false, is_cand = false;
        key[k] = 0;
        if (j < n && j >= sink_blocks && j < tail_first) {
            key[k] = order_key(v[k]);
            const uint32_t bin = key[k] >> kHistShift;
            is_def = bin > bstar;
            is_cand = bin == bstar;
        }
        md[k] = __ballot(is_def);
        mc[k] = __ballot(is_cand);
        nd += (uint32_t)__popcll(md[k]);
        nc += (uint32_t)__popcll(mc[k]);
    }
    uint32_t bd = 0, bc = 0;
    if (lane == 0) {
        bd = nd ? atomicAdd(&sh_u[2], nd) : 0u;
        bc = nc ? atomicAdd(&sh_u[3], nc) : 0u;
    }
    bd = __shfl(bd, 0);
    bc = __shfl(bc, 0);
#pragma unroll
    for (int k = 0; k < kCollectPer; k++) {
        const int j = j0 + k * kCollectThreads + tid;
        if ((md[k] >> lane) & 1ull)
            my_def[bd + __popcll(md[k] & lt)] = j;                  // at most kSliceBlocks items per slice
        if ((mc[k] >> lane) & 1ull)
            my_cand[bc + __popcll(mc[k] & lt)] = ((uint64_t)key[k] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        bd += (uint32_t)__popcll(md[k]);
        bc += (uint32_t)__popcll(mc[k]);
    }
    __syncthreads();
    if (tid == 0) {
        slot_count[2 * slot] = sh_u[2];
        slot_count[2 * slot + 1] = sh_u[3];
    }
}

// Index of the slot whose [off[s], off[s+1]) range holds p (off ascending, off[0] = 0).
__device__ __forceinline__ int slot_of(const uint32_t *off, int ns, uint32_t p)
{
    int lo = 0, hi = ns - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= p)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Grid (B, layers).
template <int N>
__global__ __launch_bounds__(kThreads) void finish_kernel(const SelectLayersT<N> Ls, const int32_t *__restrict__ ctx_len,
                                                          int max_ctx, int n_slices, int K, int sink_blocks,
                                                          int tail_tokens)
{
    const SelectWs &ws = Ls.ws[blockIdx.y];
    const uint32_t *__restrict__ slot_count = ws.slot_count;
    const int32_t *__restrict__ slot_def = ws.slot_def;
    const uint64_t *__restrict__ slot_cand = ws.slot_cand;
    uint64_t *__restrict__ spill = ws.spill;
    const int64_t spill_stride = ws.spill_stride;
    int32_t *__restrict__ sel = Ls.sel[blockIdx.y];
    int32_t *__restrict__ n_sel = Ls.n_sel[blockIdx.y];
    int32_t *__restrict__ n_tok = Ls.n_tok[blockIdx.y];
    extern __shared__ uint64_t smem64[];
    uint64_t *cand = smem64;                                            // [kCandCap]
    int32_t *defl = reinterpret_cast<int32_t *>(smem64 + kCandCap);     // [kDefCap]
    uint32_t *work = reinterpret_cast<uint32_t *>(defl + kDefCap);      // [kWorkWords]
    __shared__ uint32_t off_d[kMaxSlices + 1], off_c[kMaxSlices + 1];
    __shared__ uint32_t sh_scan[kThreads / 64];
    __shared__ uint32_t sh_u[8];   // 0,1: crossing digit / count above; 4,5: T64; 6: partial last block taken

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t L_raw = ctx_len[b];
    const int64_t r0 = ws.row0 ? ws.row0[b] : 0;
    const int L = select_len(L_raw, r0, max_ctx, ws);
    const int n = (L + kBT - 1) / kBT;
    int32_t *sel_b = sel + (int64_t)b * K;
    int tail_first = n;
    const int r = rest_to_take(L, n, K, sink_blocks, tail_tokens, &tail_first);
    if (tid == 0 && clamp_ctx(L_raw, max_ctx) != L_raw)
        raise_flag(ws.flags, QSA_FLAG_BAD_CTX_LEN);

    if (r < 0) {
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
    if (tid == 0)
        sh_u[6] = 0;

    // ---- gather the slots: prefix offsets, then one entry per thread ---------
    const int ns = r > 0 ? (n + kSliceBlocks - 1) / kSliceBlocks : 0;
    uint32_t cd = 0, cc = 0;
    if (tid < ns) {
        const int64_t slot = (int64_t)b * n_slices + tid;
        cd = slot_count[2 * slot];
        cc = slot_count[2 * slot + 1];
    }
    uint32_t tot_d, tot_c;
    const uint32_t incl_d = block_inclusive_scan<kThreads>(cd, sh_scan, &tot_d);
    const uint32_t incl_c = block_inclusive_scan<kThreads>(cc, sh_scan, &tot_c);
    if (tid < ns) {
        off_d[tid] = incl_d - cd;
        off_c[tid] = incl_c - cc;
    }
    __syncthreads();
    // Lists built from the same scores as the histogram give D < r <= D + C;
    // the clamps only keep every index in bounds.
    const uint32_t D = min(tot_d, (uint32_t)r);
    const uint32_t C = (uint32_t)min((int64_t)tot_c, spill_stride);
    const uint32_t need = min((uint32_t)r - D, C);
    uint64_t *spill_b = spill + (int64_t)b * spill_stride;
    for (uint32_t p = tid; p < D; p += kThreads) {
        const int s = slot_of(off_d, ns, p);
        defl[p] = slot_def[((int64_t)b * n_slices + s) * kSliceBlocks + (p - off_d[s])];
    }
    for (uint32_t p = tid; p < C; p += kThreads) {
        const int s = slot_of(off_c, ns, p);
        const uint64_t c = slot_cand[((int64_t)b * n_slices + s) * kSliceBlocks + (p - off_c[s])];
        if (p < (uint32_t)kCandCap)
            cand[p] = c;
        else
            spill_b[p] = c;          // read back below by this workgroup only
    }
    __syncthreads();

    // ---- choose: threshold composite T64, chosen(i) <=> comp_i >= T64 -------
    // Radix select over the composites below the shared 12-bit bin, 11 bits
    // at a time: each pass histograms the next digit of the candidates that
    // still match the prefix and keeps the bin where the count of larger ones
    // crosses `want`. A pass usually isolates the answer (a 12-bit bin spreads
    // its few hundred candidates over the next 11 bits); once the crossing bin
    // holds exactly the items still wanted, or few enough, it finishes at once.
    uint64_t T64 = ~0ull;
    if (need > 0 && need == C) {
        T64 = 0;
    } else if (need > 0) {
        auto cand_at = [&](uint32_t i) -> uint64_t { return i < (uint32_t)kCandCap ? cand[i] : spill_b[i]; };
        // the candidates share the histogram bin: the composite's top kHistBits bits
        uint64_t pmask = ((1ull << kHistBits) - 1ull) << (64 - kHistBits);
        uint64_t prefix = cand[0] & pmask;
        uint32_t want = need;
        int shift = 64 - kHistBits;
        uint32_t *h = work;                         // 2048-bin histogram
        bool done = false;
        while (!done) {
            const int bits = shift >= kDigitBits ? kDigitBits : shift;
            shift -= bits;
            const uint32_t dmask = (1u << bits) - 1u;
            for (int i = tid; i < kDigitBins; i += kThreads)
                h[i] = 0;
            __syncthreads();
            for (uint32_t i = tid; i < C; i += kThreads) {
                const uint64_t c = cand_at(i);
                if ((c & pmask) == prefix)
                    atomicAdd(&h[(c >> shift) & dmask], 1u);
            }
            __syncthreads();
            find_crossing<kDigitBins / kThreads, kThreads>(h, want, sh_scan, &sh_u[0], &sh_u[1]);
            const uint32_t digit = sh_u[0];
            const uint32_t in_bin = h[digit];
            want -= sh_u[1];
            prefix |= (uint64_t)digit << shift;
            pmask |= (uint64_t)dmask << shift;
            if (in_bin == want || shift == 0) {
                // every remaining match is chosen (or the prefix is complete)
                T64 = prefix;
                done = true;
            } else if (in_bin <= (uint32_t)kThreads) {
                // few left: rank them directly, one thread each
                uint32_t *lst_n = &sh_u[2];
                uint64_t *lst = reinterpret_cast<uint64_t *>(work + kDigitBins);   // [kThreads]
                if (tid == 0)
                    *lst_n = 0;
                __syncthreads();
                for (uint32_t i = tid; i < C; i += kThreads) {
                    const uint64_t c = cand_at(i);
                    if ((c & pmask) == prefix)
                        lst[atomicAdd(lst_n, 1u)] = c;
                }
                __syncthreads();
                const uint32_t m = *lst_n;
                if (tid < m) {
                    const uint64_t ci = lst[tid];
                    uint32_t rank = 0;
                    for (uint32_t j = 0; j < m; j++)
                        rank += lst[j] > ci ? 1u : 0u;
                    if (rank == want - 1) {         // the want-th largest of the bin
                        sh_u[4] = (uint32_t)(ci >> 32);
                        sh_u[5] = (uint32_t)ci;
                    }
                }
                __syncthreads();
                T64 = ((uint64_t)sh_u[4] << 32) | sh_u[5];
                done = true;
            }
            __syncthreads();
        }
    }

    // ---- ascending output through a bitmap, segment by segment -------------
    uint32_t *bm = work;
    uint32_t written = 0;
    const int s_end = min(sink_blocks, n);
    const int t_begin = max(tail_first, s_end);
    for (int seg0 = 0; seg0 < n; seg0 += kSegBlocks) {
        const int seg1 = min(seg0 + kSegBlocks, n);
        const int nw = (seg1 - seg0 + 31) / 32;
        __syncthreads();
        for (int i = tid; i < nw; i += kThreads)
            bm[i] = 0;
        __syncthreads();
        // forced blocks: [0, s_end) and [t_begin, n)
        for (int j = seg0 + tid; j < min(seg1, s_end); j += kThreads)
            atomicOr(&bm[(j - seg0) >> 5], 1u << ((j - seg0) & 31));
        for (int j = max(seg0, t_begin) + tid; j < seg1; j += kThreads)
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
        uint32_t pos = written + block_inclusive_scan<kThreads>(cnt, sh_scan, &total) - cnt;
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
        const int nsel = (int)min(written, (uint32_t)K);
        n_sel[b] = nsel;
        if (n_tok) {
            int nt = nsel * kBT;
            const int last_len = L - (n - 1) * kBT;
            if (last_len < kBT && sh_u[6])
                nt -= kBT - last_len;     // the partial last block is selected
            n_tok[b] = nt;
        }
    }
}

// One workgroup of kOneThreads per (sequence, layer): grid (B, layers). For
// sequences of at most kOneThreads * PER blocks the whole selection runs in
// one kernel, with every block score of the sequence held in registers
// (thread t holds blocks t + kOneThreads * i, i < PER):
//  1. the histogram copies and all block scores are requested together, the
//     scores clamped to the largest context, so one round trip brings both;
//  2. the 12-bit histogram gives the threshold bin; radix passes over the
//     scores still inside the threshold prefix (11-bit digits of the order
//     key, LDS histograms) refine it until the crossing bin holds exactly
//     the blocks still wanted, or the key is complete;
//  3. if the key is complete and only m of the blocks sharing it are wanted,
//     the m with the lowest indices are taken: their ranks come from a
//     bitmap of the equal keys and its per-word prefix counts;
//  4. the forced and chosen blocks form a bitmap (one ballot per wave gives
//     64 consecutive bits), written out in ascending order by an ordered
//     compaction.
// The result is the same set as collect_kernel + finish_kernel give.
constexpr int kOneThreads = 1024;
// Longest sequence of the one-kernel route: kOneThreads * kOneMaxPer blocks
// (65,536 tokens). Past that one CU cannot bring the scores in fast enough:
// at 65,536 blocks (256 KB of scores) the kernel took 26.7 us per layer,
// against 13.7 us for collect_kernel + finish_kernel.
constexpr int kOneMaxPer = 16;

template <int N, int PER>
__global__ __launch_bounds__(kOneThreads) void select_one_kernel(const SelectLayersT<N> Ls, int64_t bs_stride,
                                                                 const int32_t *__restrict__ ctx_len, int max_ctx,
                                                                 int K, int sink_blocks, int tail_tokens)
{
    static_assert(PER >= 1 && PER <= 64 && (PER & (PER - 1)) == 0, "a power of two up to 64");
    constexpr int kWords = kOneThreads * PER / 32;  // bitmap words over the sequence's blocks
    constexpr int WPT = PER >= 32 ? PER / 32 : 1;   // words per thread in the ordered compaction
    const bool owns_words = WPT * threadIdx.x < kWords;   // threads past the bitmap own none
    static_assert(kWords <= kDigitBins, "word prefixes reuse the digit histogram");
    const float *__restrict__ block_scores = Ls.bs[blockIdx.y];
    const uint32_t *__restrict__ hist = Ls.ws[blockIdx.y].hist;
    int32_t *__restrict__ sel = Ls.sel[blockIdx.y];
    int32_t *__restrict__ n_sel = Ls.n_sel[blockIdx.y];
    int32_t *__restrict__ n_tok = Ls.n_tok[blockIdx.y];
    __shared__ __attribute__((aligned(16))) uint32_t bm[kWords];   // equal-key bitmap, then the selection
    __shared__ uint32_t dh[kDigitBins];             // digit histogram, then per-word prefix counts
    __shared__ uint32_t sh_scan[kOneThreads / 64];
    __shared__ uint32_t sh_u[4];                    // crossing bin / count above / count in the bin

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nmax = (max_ctx + kBT - 1) / kBT;     // > K >= 1 (host), and <= bs_stride

    // One round of loads: the length, the index row offset, the histogram
    // copies, every score.
    const SelectWs &ws = Ls.ws[blockIdx.y];
    const int32_t Lraw = ctx_len[b];
    const int64_t r0 = ws.row0 ? ws.row0[b] : 0;
    constexpr int W = kHistBins / kOneThreads;
    const uint32_t *hb = hist + ((int64_t)b * kHistReps * kHistBins + W * (kOneThreads - 1 - tid));
    uint32_t hraw[kHistReps][W];
#pragma unroll
    for (int c = 0; c < kHistReps; c++)
#pragma unroll
        for (int i = 0; i < W; i++)
            hraw[c][i] = hb[c * kHistBins + i];
    const float *row = block_scores + (int64_t)b * bs_stride;
    uint32_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; i++)
        key[i] = __float_as_uint(row[min(tid + kOneThreads * i, nmax - 1)]);

    const int L = select_len(Lraw, r0, max_ctx, ws);
    const int n = (L + kBT - 1) / kBT;
    int32_t *sel_b = sel + (int64_t)b * K;
    if (tid == 0 && clamp_ctx(Lraw, max_ctx) != Lraw)
        raise_flag(ws.flags, QSA_FLAG_BAD_CTX_LEN);
    int tail_first = n;
    const int r = rest_to_take(L, n, K, sink_blocks, tail_tokens, &tail_first);
    if (r < 0) {
        // Every block fits in the budget.
        for (int j = tid; j < K; j += kOneThreads)
            sel_b[j] = j < n ? j : -1;
        if (tid == 0) {
            n_sel[b] = n;
            if (n_tok)
                n_tok[b] = L;
        }
        return;
    }

    // Blocks outside [first_el, end_el) are forced or past the sequence. A
    // block that is not eligible gets key 0, which never matches a threshold
    // prefix: keys below 2^20 (histogram bin 0) are NaN codes, so for scores
    // that are numbers the threshold bin, and with it pfx, is above 0.
    const int first_el = min(sink_blocks, n);
    const int end_el = max(tail_first, first_el);
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int j = tid + kOneThreads * i;
        const bool el = j >= first_el && j < end_el;
        key[i] = el ? order_key(__uint_as_float(key[i])) : 0u;
    }

    // ---- the threshold: chosen <=> key's prefix above pfx, or equal to it
    //      (and, on a complete key with ties, among the m lowest indices) ----
    uint32_t pfx = 0xFFFFFFFFu, pmask = 0xFFFFFFFFu;
    bool pick = r > 0;                              // some non-forced blocks are taken
    bool tie = false;
    uint32_t m = 0;
    if (r > 0) {
        uint32_t hv[W];
#pragma unroll
        for (int i = 0; i < W; i++) {
            hv[i] = 0;
#pragma unroll
            for (int c = 0; c < kHistReps; c++)
                hv[i] += hraw[c][i];
        }
        if (tid == 0) {
            sh_u[0] = kHistBins;                    // no crossing: nothing is chosen
            sh_u[1] = 0;
            sh_u[2] = 0;
        }
        __syncthreads();
        crossing_of<W, kOneThreads>(hv, (uint32_t)r, sh_scan, &sh_u[0], &sh_u[1], &sh_u[2]);
        uint32_t want = (uint32_t)r - sh_u[1];
        uint32_t in_bin = sh_u[2];
        pfx = sh_u[0] << kHistShift;
        pmask = ~0u << kHistShift;
        int shift = kHistShift;
        if (sh_u[0] >= (uint32_t)kHistBins) {       // histogram inconsistent with the lengths: take none
            pick = false;
            in_bin = 0;
            want = 0;
        }
        __syncthreads();
        while (in_bin != want && shift > 0) {       // uniform
            const int bits = shift >= kDigitBits ? kDigitBits : shift;
            shift -= bits;
            const uint32_t dmask = (1u << bits) - 1u;
            for (int i = tid; i < kDigitBins; i += kOneThreads)
                dh[i] = 0;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < PER; i++)
                if ((key[i] & pmask) == pfx)
                    atomicAdd(&dh[(key[i] >> shift) & dmask], 1u);
            __syncthreads();
            find_crossing<kDigitBins / kOneThreads, kOneThreads>(dh, want, sh_scan, &sh_u[0], &sh_u[1]);
            const uint32_t digit = sh_u[0];
            in_bin = dh[digit];
            want -= sh_u[1];
            pfx |= digit << shift;
            pmask |= dmask << shift;
            __syncthreads();
        }
        tie = in_bin != want;                       // complete key, only `want` of its blocks taken
        m = want;
    }

    if (tie) {
        // Equal keys in ascending block order: bitmap, per-word prefix, rank.
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const uint64_t bal = __ballot(key[i] == pfx);
            if (lane == 0)
                *reinterpret_cast<uint64_t *>(&bm[(kOneThreads * i + 64 * wave) >> 5]) = bal;
        }
        __syncthreads();
        uint32_t cnt = 0;
#pragma unroll
        for (int w = 0; w < WPT; w++)
            cnt += owns_words ? __popc(bm[WPT * tid + w]) : 0u;
        uint32_t total;
        uint32_t pos = block_inclusive_scan<kOneThreads>(cnt, sh_scan, &total) - cnt;
        if (owns_words) {
#pragma unroll
            for (int w = 0; w < WPT; w++) {
                dh[WPT * tid + w] = pos;
                pos += __popc(bm[WPT * tid + w]);
            }
        }
        __syncthreads();
    }

    // ---- the selection bitmap: forced blocks and chosen ones ----------------
    // A wave's ballot of round i covers words 32 i + 2 wave and + 1, which
    // hold only this wave's blocks of that round: the equal-key bits read
    // for them are never read again, so each round overwrites its own words.
    if (!pick) {                                    // uniform: only this keeps key-0 blocks out
        pfx = 0xFFFFFFFFu;
        pmask = 0u;
    }
    uint32_t last_taken = 0;
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int j = tid + kOneThreads * i;
        const uint32_t kp = key[i] & pmask;
        bool take = kp > pfx || (kp == pfx && !tie);
        if (tie) {                                  // uniform
            const uint32_t wd = (uint32_t)j >> 5;
            const uint32_t rank = dh[wd] + __popc(bm[wd] & ((1u << (j & 31)) - 1u));
            take = take || (kp == pfx && rank < m);
        }
        take = j < n && (take || j < first_el || j >= end_el);
        last_taken = j == n - 1 ? (uint32_t)take : last_taken;
        const uint64_t bal = __ballot(take);
        if (lane == 0)
            *reinterpret_cast<uint64_t *>(&bm[(kOneThreads * i + 64 * wave) >> 5]) = bal;
    }
    __syncthreads();

    // ---- ordered compaction: thread t owns words [WPT t, WPT t + WPT) -------
    uint32_t cnt = 0;
#pragma unroll
    for (int w = 0; w < WPT; w++)
        cnt += owns_words ? __popc(bm[WPT * tid + w]) : 0u;
    uint32_t total;
    uint32_t pos = block_inclusive_scan<kOneThreads>(cnt, sh_scan, &total) - cnt;
#pragma unroll
    for (int w = 0; w < WPT; w++) {
        uint32_t mw = owns_words ? bm[WPT * tid + w] : 0u;
        while (mw) {
            const int bit = __ffs(mw) - 1;
            mw &= mw - 1;
            if (pos < (uint32_t)K)
                sel_b[pos] = 32 * (WPT * tid + w) + bit;
            pos++;
        }
    }
    for (int p = (int)total + tid; p < K; p += kOneThreads)
        sel_b[p] = -1;
    if (tid == (n - 1) % kOneThreads) {
        const int nsel = (int)min(total, (uint32_t)K);
        n_sel[b] = nsel;
        if (n_tok) {
            int nt = nsel * kBT;
            const int last_len = L - (n - 1) * kBT;
            if (last_len < kBT && last_taken)
                nt -= kBT - last_len;               // the partial last block is selected
            n_tok[b] = nt;
        }
    }
}

} // namespace

template <int N>
static hipError_t launch_select_n(const SelectLayersT<N> &L, int n_layers, int64_t bs_stride, const int32_t *ctx_len,
                                  int batch, int max_ctx, int budget_blocks, int sink_blocks, int tail_tokens,
                                  hipStream_t s)
{
    const int n_blk_max = (max_ctx + kBT - 1) / kBT;
    const int n_slices = n_blk_max > 0 ? (n_blk_max + kSliceBlocks - 1) / kSliceBlocks : 1;
    if (n_blk_max > budget_blocks && n_blk_max <= kOneThreads * kOneMaxPer) {
        // the whole selection in one kernel, one workgroup per (sequence, layer)
        dim3 grid((unsigned)batch, (unsigned)n_layers);
        if (n_blk_max <= kOneThreads * 2)
            hipLaunchKernelGGL((select_one_kernel<N, 2>), grid, dim3(kOneThreads), 0, s, L, bs_stride, ctx_len,
                               max_ctx, budget_blocks, sink_blocks, tail_tokens);
        else
            hipLaunchKernelGGL((select_one_kernel<N, kOneMaxPer>), grid, dim3(kOneThreads), 0, s, L, bs_stride,
                               ctx_len, max_ctx, budget_blocks, sink_blocks, tail_tokens);
        return hipGetLastError();
    }
    if (n_blk_max > budget_blocks) {
        dim3 grid((unsigned)n_slices, (unsigned)batch, (unsigned)n_layers);
        hipLaunchKernelGGL((collect_kernel<N>), grid, dim3(kCollectThreads), 0, s, L, bs_stride, ctx_len, max_ctx,
                           n_slices, budget_blocks, sink_blocks, tail_tokens);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((finish_kernel<N>), dim3((unsigned)batch, (unsigned)n_layers), dim3(kThreads), kSmemBytes, s,
                       L, ctx_len, max_ctx, n_slices, budget_blocks, sink_blocks, tail_tokens);
    return hipGetLastError();
}

hipError_t launch_select_layers(const SelectLayers &L, int n_layers, int64_t bs_stride, const int32_t *ctx_len,
                                int batch, int max_ctx, int budget_blocks, int sink_blocks, int tail_tokens,
                                hipStream_t s)
{
    if (n_layers < 1 || n_layers > kMaxChainLayers)
        return hipErrorInvalidValue;
    if (n_layers > 1)
        return launch_select_n(L, n_layers, bs_stride, ctx_len, batch, max_ctx, budget_blocks, sink_blocks,
                               tail_tokens, s);
    const SelectLayersT<1> L1 = {{L.bs[0]}, {L.ws[0]}, {L.sel[0]}, {L.n_sel[0]}, {L.n_tok[0]}};
    return launch_select_n(L1, 1, bs_stride, ctx_len, batch, max_ctx, budget_blocks, sink_blocks, tail_tokens, s);
}

hipError_t launch_select(const float *block_scores, int64_t bs_stride, const int32_t *ctx_len, int batch,
                         int max_ctx, const SelectWs &ws, int budget_blocks, int sink_blocks, int tail_tokens,
                         int32_t *sel, int32_t *n_sel, int32_t *n_tok, hipStream_t s)
{
    SelectLayers L = {};
    L.bs[0] = block_scores;
    L.ws[0] = ws;
    L.sel[0] = sel;
    L.n_sel[0] = n_sel;
    L.n_tok[0] = n_tok;
    return launch_select_layers(L, 1, bs_stride, ctx_len, batch, max_ctx, budget_blocks, sink_blocks, tail_tokens,
                                s);
}

} // namespace qsa
