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
//  - sequences of up to kOneMaxBlocks blocks (65,536 tokens): select_one_kernel
//    holds all of a sequence's scores in one workgroup's registers, counts
//    them into a 12-bit histogram of the key's top bits and selects in one
//    launch (radix passes over the registers, and an equal-key bitmap for
//    the ties of the last key);
//  - longer sequences: each scoring workgroup leaves a candidate list of
//    its chunk's best blocks (build_chunk_list: every eligible block of the
//    chunk whose key bin is at least the list's threshold bin, some m of
//    them or more). pool_select_kernel, one workgroup per (sequence, layer),
//    gathers the lists into one pool, finds the r-th largest composite T_U of
//    the pool (r = K - |F|), and then re-reads only the chunks that could
//    still hide a block of the answer: a chunk whose list is incomplete,
//    whose every entry is at least T_U, and whose threshold lies above T_U.
//    Their missing blocks at or above T_U join the pool, and the r-th largest
//    of the pool is the exact threshold. A re-read chunk's block scores come
//    from memory when they were stored (the standalone call; in the decode
//    step, a chunk whose list was cut short by a crowded bin), and are
//    otherwise computed again from the index with the scan's own arithmetic.
//    Why this is exact: a block x of the answer missing from the pool sits in
//    a chunk whose list entries all beat it (their bins are higher), so they
//    are in the answer too, and so among the pool's best r (the pool is a
//    subset of all blocks); and x itself beats the pool's r-th largest T_U,
//    since the answer's threshold is at least T_U -- which is the test above.
//    A chunk is re-read only if its whole list is among the pool's best r,
//    so with lists of m entries at most r / m chunks are re-read.
// The selection is written in ascending order through an LDS bitmap, so the
// output needs no sort.
// Nothing is shared between workgroups inside a kernel: no global atomics on
// a few hot addresses (they serialise at the memory side) and no
// device-scope fences (on gfx950 one writes back and invalidates the XCD's
// L2). The kernel boundary after the scan orders the lists. One launch may
// cover several layers (grid y): their pointers travel in the kernel
// arguments.
#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kThreads = 1024;                     // pool_select_kernel
constexpr int kCandCap = kPoolSlots;               // pool entries held in LDS (64 KB)
constexpr int kTileBlocks = 64 / kBT;              // blocks of a 64-token scoring tile
constexpr int kLoadBatch = 4;                      // re-read loads a thread keeps in flight per round
constexpr int kSegBlocks = 1 << 18;                // bitmap segment (32 KB of LDS)
constexpr int kSegWords = kSegBlocks / 32;
constexpr int kDigitBits = 11;                     // radix digit of the pool selection
constexpr int kDigitBins = 1 << kDigitBits;        // 2048 bins, 2 per thread
constexpr int kRankDirect = 64;                    // entries ranked one per thread (each reads all)
constexpr int kCoarse = 64;                        // coarse bins of a digit histogram (one per lane)
constexpr int kPerCoarse = kDigitBins / kCoarse;   // 32 digits each
static_assert(kMaxListChunks <= kThreads, "one selection thread per chunk");

// Number of non-forced blocks to take, or -1 when every block fits.
__device__ __forceinline__ int rest_to_take(int L, int n, int K, int sink_blocks, int tail_tokens, int *tail_first)
{
    if (n <= K)
        return -1;
    *tail_first = tail_first_block(L, tail_tokens, n);
    return K - forced_count(n, sink_blocks, *tail_first);   // host guarantees >= 0
}

// Wave 0 of a workgroup: the bin of a kDigitBins-bin histogram h where the
// count from the top first reaches want (<= the histogram's total); writes
// the bin, the count above it and the count in it to out[0..2]. Two steps of
// one wave: each lane sums 32 consecutive bins and the wave finds the
// coarse bin, then the bin within it.
__device__ void wave_crossing(const uint32_t *h, uint32_t want, uint32_t *out)
{
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
    const int lane = threadIdx.x & 63;
    const u32x4_t *hv = reinterpret_cast<const u32x4_t *>(h + (kCoarse - 1 - lane) * kPerCoarse);
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < kPerCoarse / 4; i++) {
        const u32x4_t x = hv[i];
        c += x.x + x.y + x.z + x.w;
    }
    uint32_t incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d);
        if (lane >= d)
            incl += o;
    }
    int f = __ffsll((unsigned long long)__ballot(incl >= want)) - 1;
    f = f < 0 ? kCoarse - 1 : f;                    // (never: want <= the total)
    const uint32_t above_c = __shfl(incl, f) - __shfl(c, f);
    const int cbin = kCoarse - 1 - f;
    const uint32_t x = lane < kPerCoarse ? h[cbin * kPerCoarse + kPerCoarse - 1 - lane] : 0u;
    uint32_t incl2 = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl2, d);
        if (lane >= d)
            incl2 += o;
    }
    incl2 += above_c;
    int f2 = __ffsll((unsigned long long)__ballot(lane < kPerCoarse && incl2 >= want)) - 1;
    f2 = f2 < 0 ? kPerCoarse - 1 : f2;
    const uint32_t in_bin = __shfl(x, f2);
    const uint32_t above = __shfl(incl2, f2) - in_bin;
    if (lane == 0) {
        out[0] = (uint32_t)(cbin * kPerCoarse + kPerCoarse - 1 - f2);
        out[1] = above;
        out[2] = in_bin;
    }
}

// The want-th largest of a set of unique nonzero 64-bit entries held by the
// workgroup's threads: each_entry(f) calls f(x) for each entry x of the
// calling thread. 1 <= want <= their number. vmax and vmin bound the entries
// (vmax = ~0, vmin = 1 when unknown): the bits above the highest one where
// they differ are common to all of them, so the search starts below those.
// Radix select from there, 11 bits at a time: each pass histograms the next
// digit of the entries that still match the prefix and keeps the bin where
// the count of larger ones crosses `want`; once the crossing bin holds
// exactly the entries still wanted, or at most kRankDirect (ranked one per
// thread, each comparing itself with all of them), it finishes at once. h
// holds two histograms (a pass counts into one while the other is cleared
// for the next pass); the first must be zero, after a barrier, when it is
// called. All threads of the workgroup call it; returns the same value in
// every thread. Uses sh_u[0..2], [4], [5], [7].
template <typename Each>
__device__ uint64_t rth_largest(Each each_entry, uint32_t want, uint64_t vmax, uint64_t vmin, uint32_t *h,
                                uint64_t *lst, uint32_t *sh_u)
{
    const int tid = threadIdx.x;
    if (vmax == vmin)
        return vmax;                                // one entry
    int shift = 64 - __clzll((long long)(vmax ^ vmin));   // bits [shift, 64) are common
    uint64_t pmask = shift >= 64 ? 0ull : ~0ull << shift;
    uint64_t prefix = vmax & pmask;
    if (tid == 0)
        sh_u[7] = 0;                                // the short list's fill
    for (int pass = 0;; pass++) {
        uint32_t *hb = h + (pass & 1) * kDigitBins, *hn = h + ((pass + 1) & 1) * kDigitBins;
        const int bits = shift >= kDigitBits ? kDigitBits : shift;
        shift -= bits;
        const uint32_t dmask = (1u << bits) - 1u;
        for (int i = tid; i < kDigitBins; i += kThreads)
            hn[i] = 0;
        each_entry([&](uint64_t c) {
            if ((c & pmask) == prefix)
                atomicAdd(&hb[(uint32_t)(c >> shift) & dmask], 1u);
        });
        __syncthreads();
        if (tid < 64)
            wave_crossing(hb, want, sh_u);
        __syncthreads();
        const uint32_t digit = sh_u[0];
        const uint32_t in_bin = sh_u[2];
        want -= sh_u[1];
        prefix |= (uint64_t)digit << shift;
        pmask |= (uint64_t)dmask << shift;
        // sh_u[0..2] are next written after the next pass's counting barrier
        if (in_bin == want || shift == 0)
            return prefix;                          // every remaining match is chosen
        if (in_bin <= (uint32_t)kRankDirect) {
            // few left: collect them, then rank them directly, one thread each
            each_entry([&](uint64_t c) {
                if ((c & pmask) == prefix) {
                    const uint32_t pos = atomicAdd(&sh_u[7], 1u);
                    if (pos < (uint32_t)kRankDirect)
                        lst[pos] = c;
                }
            });
            __syncthreads();
            const uint32_t m = min(sh_u[7], (uint32_t)kRankDirect);
            if (tid < (int)m) {
                const uint64_t ci = lst[tid];
                uint32_t rank = 0;
                for (uint32_t j = 0; j < m; j++)
                    rank += lst[j] > ci ? 1u : 0u;
                if (rank == want - 1) {             // the want-th largest of the bin
                    sh_u[4] = (uint32_t)(ci >> 32);
                    sh_u[5] = (uint32_t)ci;
                }
            }
            __syncthreads();
            return ((uint64_t)sh_u[4] << 32) | sh_u[5];
        }
    }
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        v += __shfl_xor(v, d);
    return v;
}

// Grid (B, layers). The pool holds every list slot of the sequence, chunk c's
// at positions c * cap .. c * cap + cap - 1, so that the headers and all slots
// come in one round of loads issued before the length is known; empty slots
// hold 0 (the scan writes 0 past each list; slots of chunks past the
// sequence are ignored), which is below every block's composite (a composite
// is 0 only for key 0 and index 2^32 - 1), so a slot's value tells whether
// it holds an entry. Blocks added by the re-read follow at n_chunks * cap. In
// the common case (no chunk to re-read) the output bitmap is marked from the
// registers that brought the lists, in the pass that checks the chunks.
template <int N>
__global__ __launch_bounds__(kThreads) void pool_select_kernel(const SelectLayersT<N> Ls, int64_t bs_stride,
                                                               const int32_t *__restrict__ ctx_len, int max_ctx,
                                                               ListGeom g, int K, int sink_blocks, int tail_tokens)
{
    const SelectWs &ws = Ls.ws[blockIdx.y];
    const float *__restrict__ block_scores = Ls.bs[blockIdx.y];
    uint64_t *__restrict__ spill = ws.spill;
    int32_t *__restrict__ sel = Ls.sel[blockIdx.y];
    int32_t *__restrict__ n_sel = Ls.n_sel[blockIdx.y];
    int32_t *__restrict__ n_tok = Ls.n_tok[blockIdx.y];
    __shared__ uint64_t cand[kCandCap];             // the pool (spilling to global memory past it)
    __shared__ __attribute__((aligned(16))) uint32_t hist[2 * kDigitBins];   // radix histograms
    __shared__ uint64_t lst[kRankDirect];           // the radix select's short list
    __shared__ uint32_t bm[kSegWords];              // the output bitmap
    __shared__ uint32_t head[kMaxListChunks];       // list headers
    __shared__ uint32_t needy[kMaxListChunks];      // chunk flags, then the re-read chunks
    __shared__ uint64_t vext[2];                    // largest and smallest list entry
    __shared__ uint32_t sh_scan[kThreads / 64];
    // 0-2: crossing; 3: pool end; 4,5: threshold; 6: last block taken; 7: short-list fill
    __shared__ uint32_t sh_u[8];
    __shared__ uint32_t sh_p;                       // list entries of the sequence
    __shared__ uint32_t sh_needy;                   // needy chunks

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int cap = g.cap;
    const int NCH = g.n_chunks;                     // <= kMaxListChunks (host)
    const uint32_t E = (uint32_t)(NCH * cap);       // list slots of a sequence
    uint64_t *spill_b = spill + (int64_t)b * ws.spill_stride;
    auto at = [&](uint32_t i) -> uint64_t { return i < (uint32_t)kCandCap ? cand[i] : spill_b[i]; };
    auto put = [&](uint32_t i, uint64_t v) {
        if (i < (uint32_t)kCandCap)
            cand[i] = v;
        else
            spill_b[i] = v;                         // read back below by this workgroup only
    };

    // ---- one round: length, index row offset, headers, every list slot ------
    const int32_t L_raw = ctx_len[b];
    const int64_t r0 = ws.row0 ? ws.row0[b] : 0;
    const bool have_lists = ws.heads != nullptr;    // uniform
    const uint32_t hd = (have_lists && tid < NCH) ? ws.heads[(int64_t)b * NCH + tid] : 0u;
    const uint64_t *lists_b = have_lists ? ws.lists + (int64_t)b * E : nullptr;
    constexpr int kSpec = kCandCap / kThreads;      // slots a thread fetches in the first round
    uint64_t v[kSpec];
#pragma unroll
    for (int e = 0; e < kSpec; e++) {
        const uint32_t p = (uint32_t)(e * kThreads + tid);
        v[e] = (have_lists && p < E) ? lists_b[p] : 0ull;
    }
    // while they arrive: the first bitmap segment, the first histograms, the
    // chunk flags and the accumulators
    for (int i = tid; i < kSegWords; i += kThreads)
        bm[i] = 0;
    for (int i = tid; i < kDigitBins; i += kThreads)
        hist[i] = 0;
    if (tid < NCH)
        needy[tid] = 1u;
    if (tid == 0) {
        vext[0] = 0ull;
        vext[1] = ~0ull;
        sh_p = 0;
        sh_needy = 0;
        sh_u[6] = 0;
    }

    const int L = select_len(L_raw, r0, max_ctx, ws);
    const int n = (L + kBT - 1) / kBT;
    int32_t *sel_b = sel + (int64_t)b * K;
    int tail_first = n;
    const int r = rest_to_take(L, n, K, sink_blocks, tail_tokens, &tail_first);
    if (tid == 0) {
        const int Lc = clamp_ctx(L_raw, max_ctx);
        if (Lc != L_raw)
            raise_flag(ws.flags, QSA_FLAG_BAD_CTX_LEN);
        if (ws.row0 && Lc > 0 && (r0 < 0 || r0 + Lc > ws.n_rows))
            raise_flag(ws.flags, QSA_FLAG_BAD_INDEX_ROWS);
    }

    if (r < 0 || !have_lists) {
        // Every block fits in the budget (the host passes no lists only then).
        for (int j = tid; j < K; j += kThreads)
            sel_b[j] = j < n ? j : -1;
        if (tid == 0) {
            n_sel[b] = min(n, K);
            if (n_tok)
                n_tok[b] = n <= K ? L : K * kBT;
        }
        return;
    }
    const int s_end = min(sink_blocks, n);          // eligible blocks: [s_end, t_begin)
    const int t_begin = max(tail_first, s_end);
    const int cb = g.chunk_blocks;
    const int nc = (n + cb - 1) / cb;               // chunks of this sequence, <= NCH
    const int seg_end0 = min(n, kSegBlocks);        // blocks of the first bitmap segment
    auto mark = [&](int j, int seg0) { atomicOr(&bm[(j - seg0) >> 5], 1u << ((j - seg0) & 31)); };

    uint64_t T = ~0ull;                             // chosen <=> pool entry >= T (r > 0)
    uint32_t C = E;                                 // pool positions in use
    bool seg0_marked = false;                       // bitmap segment 0 holds the answer
    if (r > 0) {
        // ---- the pool: entries of the sequence's chunks, 0 elsewhere; its
        //      size and extremes, all from the slots' values ----------------
        if (tid < NCH)
            head[tid] = tid < nc ? hd : 0u;
        const uint32_t E_seq = (uint32_t)(nc * cap);   // slots of this sequence's chunks
        uint64_t lmax = 0ull, lmin = ~0ull;         // this thread's entries
        uint32_t cnt = 0;
        auto place = [&](uint32_t p, uint64_t x) -> bool {
            const bool valid = p < E_seq && x != 0ull;
            if (valid) {
                lmax = x > lmax ? x : lmax;
                lmin = x < lmin ? x : lmin;
                cnt++;
            }
            put(p, valid ? x : 0ull);
            return valid;
        };
        uint32_t vmask = 0;                         // which of v[] are list entries
#pragma unroll
        for (int e = 0; e < kSpec; e++) {
            const uint32_t p = (uint32_t)(e * kThreads + tid);
            if (p < E && place(p, v[e]))
                vmask |= 1u << e;
        }
        for (uint32_t p = kCandCap + tid; p < E; p += kThreads)   // more slots than the LDS pool holds
            place(p, lists_b[p]);
        const uint32_t cw = wave_sum(cnt);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const uint64_t omax = __shfl_xor(lmax, d), omin = __shfl_xor(lmin, d);
            lmax = omax > lmax ? omax : lmax;
            lmin = omin < lmin ? omin : lmin;
        }
        if (lane == 0) {
            if (cw)
                atomicAdd(&sh_p, cw);
            atomicMax(reinterpret_cast<unsigned long long *>(&vext[0]), (unsigned long long)lmax);
            atomicMin(reinterpret_cast<unsigned long long *>(&vext[1]), (unsigned long long)lmin);
        }
        __syncthreads();
        const uint32_t P = sh_p;

        // ---- T_U = the pool's r-th largest (every list entry if the pool has
        //      fewer than r). Then, in one pass over the entries: a list with
        //      an entry below T_U is not needy, and the entries at or above
        //      T_U and the forced blocks go into the bitmap, the answer unless
        //      a chunk turns out needy ------------------------------------
        const bool bounded = P >= (uint32_t)r;
        auto pool_entries = [&](auto f) {           // this thread's list entries
#pragma unroll
            for (int e = 0; e < kSpec; e++)
                if ((vmask >> e) & 1u)
                    f(v[e]);
            for (uint32_t p = kCandCap + tid; p < E; p += kThreads) {
                const uint64_t c = at(p);
                if (c != 0ull)
                    f(c);
            }
        };
        const uint64_t TU = bounded ? rth_largest(pool_entries, (uint32_t)r, vext[0], vext[1], hist, lst, sh_u) : 1ull;
#pragma unroll
        for (int e = 0; e < kSpec; e++) {
            if ((vmask >> e) & 1u) {
                if (v[e] < TU)
                    needy[(uint32_t)(e * kThreads + tid) / (uint32_t)cap] = 0u;
                else if (composite_block(v[e]) < seg_end0)
                    mark(composite_block(v[e]), 0);
            }
        }
        for (uint32_t p = kCandCap + tid; p < E; p += kThreads) {
            const uint64_t c = at(p);
            if (c != 0ull && c < TU)
                needy[p / (uint32_t)cap] = 0u;
            else if (c != 0ull && composite_block(c) < seg_end0)
                mark(composite_block(c), 0);
        }
        for (int j = tid; j < s_end; j += kThreads)
            if (j < seg_end0)
                mark(j, 0);
        for (int j = t_begin + tid; j < seg_end0; j += kThreads)
            mark(j, 0);
        __syncthreads();
        // a chunk is needy if its list is incomplete, every entry of it is at
        // least T_U, and its threshold lies above T_U (every chunk with an
        // incomplete list when the pool is short)
        bool maybe = false;
        if (tid < nc) {
            maybe = !(hd & kListComplete);
            if (bounded)
                maybe = maybe && needy[tid] && ((uint64_t)list_bin(hd) << kHistShift) > (TU >> 32);
        }
        const uint64_t nb = __ballot(maybe);
        if (lane == 0 && nb)
            atomicAdd(&sh_needy, (uint32_t)__popcll(nb));
        __syncthreads();
        const uint32_t n_needy = sh_needy;
        T = TU;
        seg0_marked = true;
        if (n_needy > 0) {
            // ---- rare: list the needy chunks, re-read them (their blocks below
            //      the list's bin that reach T_U join the pool), then the r-th
            //      largest of the pool is the threshold --------------------
            seg0_marked = false;
            const uint32_t mine = maybe ? 1u : 0u;
            uint32_t tot;
            const uint32_t pos = block_inclusive_scan<kThreads>(mine, sh_scan, &tot) - mine;
            if (mine)
                needy[pos] = (uint32_t)tid;
            for (int i = tid; i < kDigitBins; i += kThreads)
                hist[i] = 0;
            if (tid == 0)
                sh_u[3] = E;
            __syncthreads();
            // a block of a needy chunk joins the pool if it lies below the
            // list's bin and reaches T_U (wave-wide: add, append position)
            auto offer = [&](int j, float x, bool in) {
                bool add = false;
                uint64_t c = 0;
                if (in) {
                    const uint32_t key = order_key(x);
                    c = composite(key, j);
                    add = (key >> kHistShift) < list_bin(head[j / cb]) && (!bounded || c >= TU);
                }
                const uint64_t bal = __ballot(add);
                uint32_t base = 0;
                if (lane == 0 && bal)
                    base = atomicAdd(&sh_u[3], (uint32_t)__popcll(bal));
                base = __shfl(base, 0);
                const uint32_t p = base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
                if (add && p < (uint32_t)ws.spill_stride)
                    put(p, c);
            };
            // a chunk's block scores are in memory unless the scan dropped them
            auto kept = [&](int c) -> bool { return !ws.keys || (head[c] & kListScoresKept); };
            const float *row = block_scores + (int64_t)b * bs_stride;
            const uint32_t items = n_needy * (uint32_t)cb;
            for (uint32_t q0 = 0; q0 < items; q0 += kThreads * kLoadBatch) {
                float x[kLoadBatch];
                int jj[kLoadBatch];
#pragma unroll
                for (int e = 0; e < kLoadBatch; e++) {
                    const uint32_t q = q0 + e * kThreads + tid;
                    jj[e] = -1;
                    x[e] = 0.0f;
                    if (q < items) {
                        const int c = (int)needy[q / cb];
                        const int j = c * cb + (int)(q % cb);
                        if (j >= s_end && j < t_begin && kept(c)) {
                            jj[e] = j;
                            x[e] = row[j];
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < kLoadBatch; e++)
                    offer(jj[e], x[e], jj[e] >= 0);
            }
            if (ws.keys) {
                // the needy chunks whose scores the scan dropped: score their
                // tokens again, a 64-token tile per wave at a time, with the
                // scan's own arithmetic (the same bits), and take each block's
                // maximum over its valid tokens as the scan does
                IdxQuery Q;
                idx_query(ws.q_idx + (int64_t)b * kIdxH * kIdxD, ws.w_idx + (int64_t)b * kIdxH, lane, Q);
                const uint8_t *kb = ws.keys + r0 * kIdxD;
                const uint16_t *sb = ws.scales + r0;
                const uint32_t tpc = (uint32_t)cb / kTileBlocks;   // tiles per chunk
                for (uint32_t tile = (uint32_t)(tid >> 6); tile < n_needy * tpc; tile += kThreads / 64) {
                    const int c = (int)needy[tile / tpc];
                    if (kept(c))
                        continue;                                   // uniform in the wave
                    const int tw = (c * cb + (int)(tile % tpc) * kTileBlocks) * kBT;
                    idx_u32x4 k[4];
                    uint16_t sc;
                    idx_tile_load(kb, sb, tw, L, lane, k, sc);
                    float x = idx_tile_score(k, sc, Q);
                    if (tw + lane >= L)
                        x = -INFINITY;
                    x = fmaxf(x, __shfl_xor(x, 1));
                    x = fmaxf(x, __shfl_xor(x, 2));
                    const int j = (tw + lane) >> 2;
                    offer(j, x, (lane & 3) == 0 && j >= s_end && j < t_begin);
                }
            }
            __syncthreads();
            C = min(sh_u[3], (uint32_t)ws.spill_stride);
            __syncthreads();
            // P valid list entries and C - E added blocks: their r-th largest
            auto all_entries = [&](auto f) {
                for (uint32_t p = tid; p < C; p += kThreads) {
                    const uint64_t c = at(p);
                    if (c != 0ull)
                        f(c);
                }
            };
            T = P + (C - E) >= (uint32_t)r ? rth_largest(all_entries, (uint32_t)r, ~0ull, 1ull, hist, lst, sh_u)
                                           : 1ull;
        }
    }

    // ---- ascending output through a bitmap, segment by segment -------------
    uint32_t written = 0;
    for (int seg0 = 0; seg0 < n; seg0 += kSegBlocks) {
        const int seg1 = min(seg0 + kSegBlocks, n);
        const int nw = (seg1 - seg0 + 31) / 32;
        if (seg0 > 0 || !seg0_marked) {
            __syncthreads();
            if (seg0 > 0 || r > 0)                  // (r == 0: still clear from the start)
                for (int i = tid; i < nw; i += kThreads)
                    bm[i] = 0;
            __syncthreads();
            // forced blocks: [0, s_end) and [t_begin, n)
            for (int j = seg0 + tid; j < min(seg1, s_end); j += kThreads)
                mark(j, seg0);
            for (int j = max(seg0, t_begin) + tid; j < seg1; j += kThreads)
                mark(j, seg0);
            if (r > 0) {
                for (uint32_t i = tid; i < C; i += kThreads) {
                    const uint64_t c = at(i);
                    if (c != 0ull && c >= T) {
                        const int j = composite_block(c);
                        if (j >= seg0 && j < seg1)
                            mark(j, seg0);
                    }
                }
            }
            __syncthreads();
        }                                           // (else: marked before the needy count's barrier)
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
//  1. all block scores are requested in one round, clamped to the largest
//     context, and counted into an LDS histogram of the keys' top 12 bits;
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
// The result is the same set as the chunk lists and pool_select_kernel give.
constexpr int kOneThreads = 1024;
// Longest sequence of the one-kernel route: kOneThreads * kOneMaxPer blocks
// (65,536 tokens). Past that one CU cannot bring the scores in fast enough:
// at 65,536 blocks (256 KB of scores) the kernel took 26.7 us per layer,
// against 13.7 us for the two-kernel route it was measured against.
constexpr int kOneMaxPer = 16;
static_assert(kOneThreads * kOneMaxPer == kOneMaxBlocks, "route boundary");

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
    int32_t *__restrict__ sel = Ls.sel[blockIdx.y];
    int32_t *__restrict__ n_sel = Ls.n_sel[blockIdx.y];
    int32_t *__restrict__ n_tok = Ls.n_tok[blockIdx.y];
    __shared__ __attribute__((aligned(16))) uint32_t bm[kWords];   // equal-key bitmap, then the selection
    __shared__ uint32_t dh[kDigitBins];             // digit histogram, then per-word prefix counts
    __shared__ uint32_t lh[kHistBins];              // 12-bit histogram of the eligible keys
    __shared__ uint32_t sh_scan[kOneThreads / 64];
    __shared__ uint32_t sh_u[4];                    // crossing bin / count above / count in the bin

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nmax = (max_ctx + kBT - 1) / kBT;     // > K >= 1 (host), and <= bs_stride

    // One round of loads: the length, the index row offset, every score.
    const SelectWs &ws = Ls.ws[blockIdx.y];
    const int32_t Lraw = ctx_len[b];
    const int64_t r0 = ws.row0 ? ws.row0[b] : 0;
    constexpr int W = kHistBins / kOneThreads;
    for (int i = tid; i < kHistBins; i += kOneThreads)
        lh[i] = 0;
    const float *row = block_scores + (int64_t)b * bs_stride;
    uint32_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; i++)
        key[i] = __float_as_uint(row[min(tid + kOneThreads * i, nmax - 1)]);

    const int L = select_len(Lraw, r0, max_ctx, ws);
    const int n = (L + kBT - 1) / kBT;
    int32_t *sel_b = sel + (int64_t)b * K;
    if (tid == 0) {
        const int Lc = clamp_ctx(Lraw, max_ctx);
        if (Lc != Lraw)
            raise_flag(ws.flags, QSA_FLAG_BAD_CTX_LEN);
        if (ws.row0 && Lc > 0 && (r0 < 0 || r0 + Lc > ws.n_rows))
            raise_flag(ws.flags, QSA_FLAG_BAD_INDEX_ROWS);
    }
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
    __syncthreads();                                // lh cleared
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int j = tid + kOneThreads * i;
        const bool el = j >= first_el && j < end_el;
        key[i] = el ? order_key(__uint_as_float(key[i])) : 0u;
        if (el && r > 0)
            atomicAdd(&lh[key[i] >> kHistShift], 1u);
    }

    // ---- the threshold: chosen <=> key's prefix above pfx, or equal to it
    //      (and, on a complete key with ties, among the m lowest indices) ----
    uint32_t pfx = 0xFFFFFFFFu, pmask = 0xFFFFFFFFu;
    bool pick = r > 0;                              // some non-forced blocks are taken
    bool tie = false;
    uint32_t m = 0;
    if (r > 0) {
        __syncthreads();                            // lh complete
        uint32_t hv[W];
#pragma unroll
        for (int i = 0; i < W; i++)
            hv[i] = lh[W * (kOneThreads - 1 - tid) + i];
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
                                  int batch, int max_ctx, const ListGeom &g, int budget_blocks, int sink_blocks,
                                  int tail_tokens, hipStream_t s)
{
    const int n_blk_max = (max_ctx + kBT - 1) / kBT;
    dim3 grid((unsigned)batch, (unsigned)n_layers);
    if (n_blk_max > budget_blocks && n_blk_max <= kOneMaxBlocks) {
        // the whole selection in one kernel, one workgroup per (sequence, layer)
        if (n_blk_max <= kOneThreads * 2)
            hipLaunchKernelGGL((select_one_kernel<N, 2>), grid, dim3(kOneThreads), 0, s, L, bs_stride, ctx_len,
                               max_ctx, budget_blocks, sink_blocks, tail_tokens);
        else
            hipLaunchKernelGGL((select_one_kernel<N, kOneMaxPer>), grid, dim3(kOneThreads), 0, s, L, bs_stride,
                               ctx_len, max_ctx, budget_blocks, sink_blocks, tail_tokens);
        return hipGetLastError();
    }
    // the chunk lists (or, when every sequence fits the budget, all blocks)
    if (uses_lists(max_ctx, budget_blocks) &&
        (g.n_chunks < 1 || g.n_chunks > kMaxListChunks || (int64_t)g.n_chunks * g.chunk_blocks < n_blk_max ||
         g.cap < 1 || g.cap > kListCap))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((pool_select_kernel<N>), grid, dim3(kThreads), 0, s, L, bs_stride, ctx_len, max_ctx, g,
                       budget_blocks, sink_blocks, tail_tokens);
    return hipGetLastError();
}

hipError_t launch_select_layers(const SelectLayers &L, int n_layers, int64_t bs_stride, const int32_t *ctx_len,
                                int batch, int max_ctx, const ListGeom &g, int budget_blocks, int sink_blocks,
                                int tail_tokens, hipStream_t s)
{
    if (n_layers < 1 || n_layers > kMaxChainLayers)
        return hipErrorInvalidValue;
    if (n_layers > 1)
        return launch_select_n(L, n_layers, bs_stride, ctx_len, batch, max_ctx, g, budget_blocks, sink_blocks,
                               tail_tokens, s);
    const SelectLayersT<1> L1 = {{L.bs[0]}, {L.ws[0]}, {L.sel[0]}, {L.n_sel[0]}, {L.n_tok[0]}};
    return launch_select_n(L1, 1, bs_stride, ctx_len, batch, max_ctx, g, budget_blocks, sink_blocks, tail_tokens,
                           s);
}

hipError_t launch_select(const float *block_scores, int64_t bs_stride, const int32_t *ctx_len, int batch,
                         int max_ctx, const SelectWs &ws, const ListGeom &g, int budget_blocks, int sink_blocks,
                         int tail_tokens, int32_t *sel, int32_t *n_sel, int32_t *n_tok, hipStream_t s)
{
    SelectLayers L = {};
    L.bs[0] = block_scores;
    L.ws[0] = ws;
    L.sel[0] = sel;
    L.n_sel[0] = n_sel;
    L.n_tok[0] = n_tok;
    return launch_select_layers(L, 1, bs_stride, ctx_len, batch, max_ctx, g, budget_blocks, sink_blocks,
                                tail_tokens, s);
}

} // namespace qsa
