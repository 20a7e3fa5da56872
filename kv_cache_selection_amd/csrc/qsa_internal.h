// qsa_internal.h -- shared constants, workspace layout and device helpers of
// libqsa (internal; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/libqsa.h"

namespace qsa {

// Compiled geometry.
constexpr int kHq = 16;          // query heads
constexpr int kHkv = 2;          // KV heads
constexpr int kGroup = kHq / kHkv;
constexpr int kDh = 256;         // head dim
constexpr int kIdxH = 4;         // indexer heads
constexpr int kIdxD = 64;        // indexer dim (e4m3 codes per key)
constexpr int kBT = 4;           // tokens per C4 block
constexpr int kRowElems = 2 * kHkv * kDh;      // bf16 values per KV row
constexpr int kRowBytes = 2 * kRowElems;       // 2048
constexpr int kMaxBudget = 8192;               // tokens
constexpr int kMaxCtx = 1 << 21;               // tokens per sequence

// Selection: 12-bit histogram of the order key's top bits.
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;

// Attention: tokens per split. A call whose kTPS-token splits number at
// least three quarters of the device's CUs uses splits of kTPS tokens;
// smaller calls use kTPSMin, so that they still spread over the CUs. The workspace holds the partial
// outputs of kTPSMin-token splits.
constexpr int kTPS = 128;
constexpr int kTPSMin = 64;

// Monotone map of a float to uint32: a < b  <=>  key(a) < key(b); -0.0 maps
// to the key of +0.0 so that the two compare equal, as floats do.
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0)
        u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int clamp_ctx(int32_t L, int max_ctx)
{
    return L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
}

// Records a contract violation (QSA_FLAG_*) in the call's flags word, if it
// has one. Only the lanes that found one execute the atomic.
__device__ __forceinline__ void raise_flag(uint32_t *flags, uint32_t bit)
{
    if (flags)
        atomicOr(flags, bit);
}

// Block j is forced when it is one of the first sink blocks or holds one of
// the last tail tokens.
__device__ __forceinline__ int tail_first_block(int L, int tail_tokens, int n_blk)
{
    if (tail_tokens <= 0)
        return n_blk;
    int first = L - tail_tokens;
    return (first < 0 ? 0 : first) / kBT;
}

__device__ __forceinline__ int forced_count(int n_blk, int sink, int tail_first)
{
    int s = sink < n_blk ? sink : n_blk;
    int t0 = tail_first > s ? tail_first : s;
    return s + (n_blk > t0 ? n_blk - t0 : 0);
}

// Scoring chunks: tokens per scoring workgroup, a multiple of 512 grown
// while the grid keeps at least 512 workgroups (2 per CU, 16 waves) per
// layer, so every CU streams. At most kMaxScoreChunkTokens; the result gives
// fewer than 1024 chunks per sequence for any batch and max_ctx <= kMaxCtx.
constexpr int kScoreWgTokens = 512;
constexpr int kMaxScoreChunkTokens = 8192;
inline int score_chunk_tokens(int batch, int max_ctx)
{
    int chunk = kScoreWgTokens;
    while (chunk < kMaxScoreChunkTokens &&
           (int64_t)batch * (((int64_t)max_ctx + 2 * chunk - 1) / (2 * chunk)) >= 512)
        chunk *= 2;
    return chunk;
}

// Candidate lists of the long-context selection. Each scoring chunk of a
// sequence keeps, from its own block scores, the eligible blocks whose key
// lies in the top histogram bins: the smallest such set of at least m
// blocks, or, when the bin that reaches m would take the list past cap
// entries, the blocks above that bin only. The selection kernel then works on
// the union of the lists, and re-reads only chunks whose whole list it took
// (their next blocks could still belong to the answer).
constexpr int kListCap = 128;                  // entries per chunk list, at most
constexpr int kMaxListChunks = 1024;           // chunks per sequence (one selection thread each)
constexpr int kPoolSlots = 8192;               // list slots the selection holds in LDS (more spill)
struct ListGeom {
    int chunk_blocks;    // blocks per chunk
    int n_chunks;        // chunks per sequence (row stride of the headers)
    int m;               // entries a list aims at
    int cap;             // entries a list may hold (row stride of the lists)
};
// m is about three times a chunk's share of the budget, and at least 8 where
// every chunk's cap = 2 m slots still fit the selection's LDS pool (else at
// least 4): a chunk whose share of the answer reaches m is then rare unless
// the scores cluster. (With a share of one block, as at 1M tokens in 512
// chunks, a floor of 4 left one to nine chunks per sequence and layer to be
// re-read: the share is about Poisson, and five or more of 512 chunks hold at
// least five of the answer's blocks on average.) cap = 2 m leaves room for
// the blocks that share the m-th block's bin; a crowded bin cuts the list
// short instead.
inline ListGeom list_geom(int batch, int max_ctx, int budget_blocks)
{
    ListGeom g;
    g.chunk_blocks = score_chunk_tokens(batch, max_ctx) / kBT;
    const int n_blk = (max_ctx + kBT - 1) / kBT;
    g.n_chunks = n_blk > 0 ? (n_blk + g.chunk_blocks - 1) / g.chunk_blocks : 1;
    const int m_floor = (int64_t)g.n_chunks * 16 <= kPoolSlots ? 8 : 4;
    int m = (int)((3 * (int64_t)budget_blocks + g.n_chunks - 1) / g.n_chunks);
    m = m < m_floor ? m_floor : (m > kListCap / 2 ? kListCap / 2 : m);
    g.m = m;
    g.cap = 2 * m;
    return g;
}
// Sequences of at most this many blocks are selected by one workgroup
// holding every score (select_one_kernel); longer ones go through the lists.
constexpr int kOneMaxBlocks = 16384;

// Header of a chunk list: entry count (bits 0-15); threshold bin (bits
// 16-28): the list holds exactly the chunk's eligible blocks whose key bin is
// at least this; bit 30: the chunk's block scores were stored; bit 31: the
// list holds every eligible block of the chunk.
constexpr uint32_t kListScoresKept = 1u << 30;
constexpr uint32_t kListComplete = 1u << 31;
__device__ __forceinline__ uint32_t list_count(uint32_t h) { return h & 0xFFFFu; }
__device__ __forceinline__ uint32_t list_bin(uint32_t h) { return (h >> 16) & 0x1FFFu; }

// Block j with order key k as a 64-bit composite: unique per block, and
// ordered like (score descending, block index ascending).
__device__ __forceinline__ uint64_t composite(uint32_t key, int j)
{
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}
__device__ __forceinline__ int composite_block(uint64_t c) { return (int)(0xFFFFFFFFu - (uint32_t)c); }

struct SelectWs {
    uint32_t *heads;       // [B][n_chunks] chunk list headers (long-context route)
    uint64_t *lists;       // [B][n_chunks][cap] chunk lists: composites
    uint64_t *spill;       // [B][spill_stride] pool entries past the selection kernel's LDS
    int64_t spill_stride;  // n_chunks * cap + blocks of the longest sequence
    uint32_t *flags;       // the call's flags word (QSA_FLAG_*), or null
    // The index rows of the batch (qsa_decode_step): a sequence whose rows
    // [row0[b], row0[b] + L) fall outside [0, n_rows) was scored as empty, and
    // the selection takes it as empty too. Null when there is no index.
    const int64_t *row0;
    int64_t n_rows;
    // The layer's index and indexer query (qsa_decode_step, whose scan keeps
    // the block scores of a list-route chunk only when its list was cut short
    // by a crowded bin): a chunk to re-read whose scores were not kept is
    // scored again from these. Null: every chunk's block scores are there.
    const uint8_t *keys;
    const uint16_t *scales;
    const uint16_t *q_idx;
    const float *w_idx;
};

// The length the selection works with: ctx_len clamped to [0, max_ctx], or 0
// for a sequence whose index rows fall outside the index buffer.
__device__ __forceinline__ int select_len(int32_t L_raw, int64_t r0, int max_ctx, const SelectWs &ws)
{
    const int L = clamp_ctx(L_raw, max_ctx);
    return (ws.row0 && (r0 < 0 || r0 + L > ws.n_rows)) ? 0 : L;
}

struct AttnWs {
    float *part_o;       // [B][kHq][n_split][kDh]; room for splits of kTPSMin tokens
    float *part_lse;     // [B][kHq][n_split]
    int tps;             // tokens per split of this call: kTPS or kTPSMin
    int n_split;         // splits per sequence: budget / tps, rounded up
    uint32_t *flags;     // the call's flags word, or null
};

// One launch of the selection or attention kernels may cover several layers
// (independent units of one step): the per-layer pointers travel in the
// kernel arguments and the layer is a grid coordinate, so a group of layers
// costs one latency chain instead of one per layer.
// A single-layer launch passes tables of one entry (N = 1), so that its
// kernel arguments stay small.
constexpr int kMaxChainLayers = 16;

template <int N>
struct ScoreLayersT {
    const uint8_t *keys[N];               // index codes [rows][kIdxD]
    const uint16_t *scales[N];            // fp16 scales [rows]
    const uint16_t *q_idx[N];             // bf16 [B][kIdxH][kIdxD]
    const float *w_idx[N];                // [B][kIdxH]
    float *token_scores[N];               // [rows] or null
    float *block_scores[N];               // [B][bs_stride]
    uint32_t *heads[N];                   // chunk list headers, or null (no lists)
    uint64_t *lists[N];                   // chunk lists
    uint32_t *flags;                      // the call's flags word, or null
    // 0: store every block score; 1 (qsa_decode_step): a chunk with a list
    // stores its block scores only when the list was cut short by a crowded
    // bin (the selection scores the other chunks it re-reads again)
    int drop_listed_bs;
};
using ScoreLayers = ScoreLayersT<kMaxChainLayers>;

template <int N>
struct GatherLayersT {
    const int32_t *sel[N];                // [B][budget_blocks]
    const int32_t *n_sel[N];              // [B]
    const int32_t *pt[N];                 // page table [B][pt_stride]
    const void *pool[N];                  // [n_slots][kRowBytes], device or mapped pinned host memory
    void *out[N];                         // staging rows [B][budget_tokens][kRowBytes]
    int32_t *n_tok[N];                    // [B] or null
    uint32_t *flags;                      // the call's flags word, or null
};
using GatherLayers = GatherLayersT<kMaxChainLayers>;

template <int N>
struct SelectLayersT {
    const float *bs[N];                   // block scores [B][bs_stride]
    SelectWs ws[N];
    int32_t *sel[N];                      // [B][budget_blocks]
    int32_t *n_sel[N];                    // [B]
    int32_t *n_tok[N];                    // [B] or null
};
using SelectLayers = SelectLayersT<kMaxChainLayers>;

template <int N>
struct AttnLayersT {
    const uint16_t *q[N];                 // [B][kHq][kDh] bf16
    const uint8_t *rows[N];               // pool rows (paged) or staged rows [B][budget_tokens]
    const int32_t *pt[N];                 // page table [B][pt_stride] (paged)
    int64_t n_slots[N];                   // rows in the pool (paged)
    const int32_t *sel[N];                // [B][budget_blocks] (paged)
    const int32_t *n_tok[N];
    float *part_o[N];
    float *part_lse[N];
    float *out[N];                        // [B][kHq][kDh] fp32
    uint32_t *flags;                      // the call's flags word, or null
};
using AttnLayers = AttnLayersT<kMaxChainLayers>;

// A physical slot read from a page table, forced into [0, n_slots) so that a
// bad entry can never address memory outside the pool.
__device__ __forceinline__ int64_t safe_slot(int32_t slot, int64_t n_slots)
{
    return ((uint64_t)(int64_t)slot < (uint64_t)n_slots) ? (int64_t)slot : 0;
}

// Block-wide inclusive prefix sum of one uint32 per thread.
template <int NT>
__device__ inline uint32_t block_inclusive_scan(uint32_t v, uint32_t *sh /* [NT / 64] */, uint32_t *total)
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
    for (int w = 0; w < NT / 64; w++) {
        const uint32_t x = sh[w];
        off += (w < wave) ? x : 0u;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return v + off;
}

// Walk a histogram of NT * W bins from the top: the bin where the running
// count first reaches `want`, the count strictly above it and the count in
// it (outputs untouched when the whole histogram holds fewer than `want`).
// Thread i holds bins W (NT - 1 - i) .. + W - 1 in hv, so thread 0 holds the
// top ones. Returns the histogram's total.
template <int W, int NT>
__device__ uint32_t crossing_of(const uint32_t (&hv)[W], uint32_t want, uint32_t *sh_scan, uint32_t *bin_out,
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
    return total;
}

// The same over a histogram in memory.
template <int W, int NT>
__device__ void find_crossing(const uint32_t *h, uint32_t want, uint32_t *sh_scan, uint32_t *bin_out,
                              uint32_t *above_out, uint32_t *in_bin_out = nullptr)
{
    const int tr = NT - 1 - threadIdx.x;
    uint32_t hv[W];
#pragma unroll
    for (int i = 0; i < W; i++)
        hv[i] = h[W * tr + i];
    crossing_of<W, NT>(hv, want, sh_scan, bin_out, above_out, in_bin_out);
}

// Largest value of v over the wave.
__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t o = __shfl_xor(v, d);
        v = o > v ? o : v;
    }
    return v;
}

// One chunk's candidate list (see ListGeom), built by the NT threads of a
// workgroup from its LDS histogram `lhist` of the eligible blocks' key bins
// (top_bin: the highest bin that holds one) and its LDS copy `lbs` of the
// chunk's block scores (blocks blk_begin .. blk_end - 1; eligible: el_begin
// <= j < el_end). Call after a barrier that completes lhist and lbs; the
// other waves' stores do not wait for the search. Wave 0 finds the bin where
// the count from the top reaches m, 64 bins at a time from top_bin (one
// step, unless the chunk's scores spread over more than 64 bins); then every
// thread places its eligible blocks at or above the list's threshold bin.
// Writes the header and the entries (in no particular order), and 0 in the
// list's unused slots, so that a reader can tell entries from empty slots by
// their value (no block's composite is 0). The header's kListScoresKept bit is
// set when keep_all is, or when the list was cut short by a crowded bin; the
// return value (the same for every thread) says whether it was, so that the
// caller stores the chunk's block scores then. `sh` is four words of LDS.
// NT >= cap.
template <int NT>
__device__ bool build_chunk_list(const uint32_t *lhist, const float *lbs, int blk_begin, int blk_end, int el_begin,
                                 int el_end, int m, int cap, int top_bin, bool keep_all, uint32_t *sh,
                                 uint32_t *head_out, uint64_t *list_out)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int lo = blk_begin > el_begin ? blk_begin : el_begin;
    const int hi = blk_end < el_end ? blk_end : el_end;
    const uint32_t n_el = hi > lo ? (uint32_t)(hi - lo) : 0u;
    if (tid < 64) {
        uint32_t theta = 0, size = n_el;
        bool complete = true, cut = false;
        if (n_el >= (uint32_t)m) {
            uint32_t carry = 0;
            for (int hb = top_bin; hb >= 0; hb -= 64) {        // uniform in the wave
                const int bin = hb - lane;                      // lane 0: the highest bin of the window
                const uint32_t h = bin >= 0 ? lhist[bin] : 0u;
                uint32_t incl = h;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const uint32_t o = __shfl_up(incl, d);
                    if (lane >= d)
                        incl += o;
                }
                incl += carry;
                const uint64_t hit = __ballot(incl >= (uint32_t)m);
                if (hit) {
                    const int f = __ffsll((unsigned long long)hit) - 1;
                    const uint32_t cum = __shfl(incl, f);
                    const uint32_t in_bin = __shfl(h, f);
                    if (cum <= (uint32_t)cap) {
                        theta = (uint32_t)(hb - f);
                        size = cum;
                        complete = cum == n_el;
                    } else {                                    // the crossing bin would overflow
                        theta = (uint32_t)(hb - f + 1);
                        size = cum - in_bin;
                        complete = false;
                        cut = true;
                    }
                    break;
                }
                carry = __shfl(incl, 63);
            }
        }
        if (size > (uint32_t)cap) {                             // never, with lhist consistent
            size = (uint32_t)cap;
            complete = false;
            cut = true;
        }
        const bool keep = keep_all || cut;
        if (tid == 0) {
            sh[0] = theta;
            sh[1] = 0;
            sh[2] = size;
            sh[3] = keep ? 1u : 0u;
            *head_out = size | (theta << 16) | (complete ? kListComplete : 0u) | (keep ? kListScoresKept : 0u);
        }
    }
    __syncthreads();
    const uint32_t theta = sh[0];
    const bool kept = sh[3] != 0u;
    if (tid >= (int)sh[2] && tid < cap)
        list_out[tid] = 0ull;
    for (int j0 = blk_begin; j0 < blk_end; j0 += NT) {
        const int j = j0 + tid;
        uint32_t key = 0;
        bool in = false;
        if (j < blk_end && j >= el_begin && j < el_end) {
            key = order_key(lbs[j - blk_begin]);
            in = (key >> kHistShift) >= theta;
        }
        const uint64_t bal = __ballot(in);
        uint32_t base = 0;
        if (lane == 0 && bal)
            base = atomicAdd(&sh[1], (uint32_t)__popcll(bal));
        base = __shfl(base, 0);
        const uint32_t pos = base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        if (in && pos < (uint32_t)cap)
            list_out[pos] = composite(key, j);
    }
    return kept;
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// Eight e4m3 codes (two dwords, lowest byte first) -> eight bf16 (exact). The
// packed results are moved as whole 32-bit words: extracting single __bf16
// elements of a pair lets the compiler duplicate the low half.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1)
{
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
    const u32x4_t v = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
    return __builtin_bit_cast(bf16x8, v);
}

// ---- the indexer's token score on the matrix cores --------------------------
// s_t = sum over the 4 heads of w_h ReLU(sigma_t (q_h . k_t)) (digest,
// mechanism section), for a tile of 64 tokens per wave. Every kernel that
// scores index rows uses these three functions, so a token's score has the
// same bits wherever it is computed (the scan, and the selection when it
// scores a chunk again).
//
// A wave scores its tile as 4 groups of 16 tokens. For group g, lane l loads
// the 16 bytes at offset 16 (l >> 4) of token 16 g + (l & 15), so each of the
// wave's four 16-byte loads reads one contiguous 1 KB piece of the tile. The
// e4m3 codes are widened to bf16 (exact) and the 4-head x 64-dim products run
// as v_mfma_f32_16x16x32_bf16 (B = 32 dims x 16 tokens): the lane's first 8
// bytes feed one MFMA chain and its last 8 the other, and the query operand A
// follows the same permutation of the dims. For group g the query heads sit in
// rows 4g..4g+3 of A (zeros elsewhere), so the four groups accumulate into
// one 16x16 tile whose row 4g+h, column j (head h of token 16g+j) the MFMA
// output layout places in lane 16g+j: each lane ends with its own token's 4
// head products. bf16 x bf16 products are exact in fp32; accumulation is
// fp32, and the epilogue's multiply-adds are explicit fused operations so
// that no kernel rounds them differently.
typedef __attribute__((ext_vector_type(4))) uint32_t idx_u32x4;
typedef __attribute__((ext_vector_type(4))) float idx_f32x4;

struct IdxQuery {
    bf16x8 qa[4][2];      // A operands: group g, first / last 8 dims of the lane's 16
    float w[kIdxH];       // head weights
};

// Sequence b's query operands: q_b = q_idx + b * 4 * 64 (bf16 bits), w_b = w_idx + b * 4.
__device__ __forceinline__ void idx_query(const uint16_t *__restrict__ q_b, const float *__restrict__ w_b, int lane,
                                          IdxQuery &Q)
{
    const idx_u32x4 *qrow = reinterpret_cast<const idx_u32x4 *>(q_b + (lane & 3) * kIdxD + 16 * (lane >> 4));
    const idx_u32x4 q0 = qrow[0], q1 = qrow[1];
    const idx_u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < 4; g++) {
        const bool mine = ((lane & 15) >> 2) == g;
        Q.qa[g][0] = __builtin_bit_cast(bf16x8, mine ? q0 : z);
        Q.qa[g][1] = __builtin_bit_cast(bf16x8, mine ? q1 : z);
    }
#pragma unroll
    for (int h = 0; h < kIdxH; h++)
        Q.w[h] = w_b[h];
}

// The lane's pieces of the tile of tokens [tw, tw + 64) of a sequence whose
// rows start at kb (codes) and sb (scales); tokens at or past L read nothing.
__device__ __forceinline__ void idx_tile_load(const uint8_t *__restrict__ kb, const uint16_t *__restrict__ sb, int tw,
                                              int L, int lane, idx_u32x4 *k, uint16_t &sc)
{
#pragma unroll
    for (int g = 0; g < 4; g++) {
        const int t = tw + 16 * g + (lane & 15);
        k[g] = t < L ? __builtin_nontemporal_load(
                           reinterpret_cast<const idx_u32x4 *>(kb + (int64_t)t * kIdxD + 16 * (lane >> 4)))
                     : idx_u32x4{0u, 0u, 0u, 0u};
    }
    sc = (tw + lane < L) ? sb[tw + lane] : (uint16_t)0;
}

// Score of token tw + lane of the tile (valid or not: the caller masks).
__device__ __forceinline__ float idx_tile_score(const idx_u32x4 *k, uint16_t sc, const IdxQuery &Q)
{
    idx_f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < 4; g++) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Q.qa[g][0], e4m3x8_to_bf16x8(k[g].x, k[g].y), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Q.qa[g][1], e4m3x8_to_bf16x8(k[g].z, k[g].w), acc1, 0, 0, 0);
    }
    const idx_f32x4 acc = acc0 + acc1;      // acc[h] = q_h . k_t
    const float sigma = (float)__builtin_bit_cast(_Float16, sc);
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < kIdxH; h++)
        s = __builtin_fmaf(Q.w[h], fmaxf(sigma * acc[h], 0.0f), s);
    return s;
}

// Kernel launchers (one translation unit each).
hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s);
hipError_t launch_copy_u32(const uint32_t *src, uint32_t *dst, int64_t n, hipStream_t s);

// True when a call's selection goes through the chunk lists (sequences
// longer than the one-workgroup route, and longer than the budget).
inline bool uses_lists(int max_ctx, int budget_blocks)
{
    const int n_blk = (max_ctx + kBT - 1) / kBT;
    return n_blk > budget_blocks && n_blk > kOneMaxBlocks;
}

// Index scoring of one layer. heads/lists null: no chunk lists.
hipError_t launch_index_score(const uint8_t *keys, const uint16_t *scales, const uint16_t *q_idx,
                              const float *w_idx, const int32_t *ctx_len, const int64_t *row0, int64_t n_rows,
                              int batch, int max_ctx, float *token_scores, float *block_scores, int64_t bs_stride,
                              uint32_t *heads, uint64_t *lists, const ListGeom &g, int budget_blocks,
                              int sink_blocks, int tail_tokens, uint32_t *flags, hipStream_t s,
                              hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr, uint32_t *clear_flags = nullptr,
                              bool drop_listed_bs = false);

// Index scoring of layers 0 .. n_layers - 1 of L in one launch (grid z =
// layer); token_scores and heads must be null for all layers or for none.
// clear_flags non-null: the launch first zeroes that flags word, and raises
// no flag itself (L.flags must then be null; the selection raises what the
// scan would have).
hipError_t launch_index_score_layers(const ScoreLayers &L, int n_layers, const int32_t *ctx_len, const int64_t *row0,
                                     int64_t n_rows, int batch, int max_ctx, int64_t bs_stride, const ListGeom &g,
                                     int budget_blocks, int sink_blocks, int tail_tokens, hipStream_t s,
                                     hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr,
                                     uint32_t *clear_flags = nullptr);

// Chunk lists built from existing block scores (standalone selection call).
hipError_t launch_list_build(const float *block_scores, int64_t bs_stride, const int32_t *ctx_len, int batch,
                             int max_ctx, uint32_t *heads, uint64_t *lists, const ListGeom &g, int budget_blocks,
                             int sink_blocks, int tail_tokens, hipStream_t s);

hipError_t launch_select(const float *block_scores, int64_t bs_stride, const int32_t *ctx_len, int batch,
                         int max_ctx, const SelectWs &ws, const ListGeom &g, int budget_blocks, int sink_blocks,
                         int tail_tokens, int32_t *sel, int32_t *n_sel, int32_t *n_tok, hipStream_t s);

// Selection of layers 0 .. n_layers - 1 of L (n_layers <= kMaxChainLayers).
hipError_t launch_select_layers(const SelectLayers &L, int n_layers, int64_t bs_stride, const int32_t *ctx_len,
                                int batch, int max_ctx, const ListGeom &g, int budget_blocks, int sink_blocks,
                                int tail_tokens, hipStream_t s);

hipError_t launch_gather(const int32_t *sel, const int32_t *n_sel, const int32_t *ctx_len, int batch, int max_ctx,
                         const int32_t *pt, int64_t pt_stride, int64_t n_slots, const void *pool, void *out, int budget_blocks,
                         int budget_tokens, int32_t *n_tok, uint32_t *flags, hipStream_t s);

// Row gathers of layers 0 .. n_layers - 1 of L in one launch (grid z = layer).
hipError_t launch_gather_layers(const GatherLayers &L, int n_layers, const int32_t *ctx_len, int batch, int max_ctx,
                                int64_t pt_stride, int64_t n_slots, int budget_blocks, int budget_tokens,
                                hipStream_t s, int max_wgs = 0);

// Attention over staged rows (kv != nullptr) or through the page table.
hipError_t launch_attention_staged(const uint16_t *q, const void *kv, const int32_t *n_tok, int batch,
                                   int budget_tokens, float sm_scale, const AttnWs &ws, float *out,
                                   hipStream_t s);

hipError_t launch_attention_paged(const uint16_t *q, const void *pool, const int32_t *pt, int64_t pt_stride,
                                  int64_t n_slots,
                                  const int32_t *sel, const int32_t *n_tok, const int32_t *ctx_len, int max_ctx,
                                  int batch, int budget_blocks, int budget_tokens, float sm_scale,
                                  const AttnWs &ws, float *out, hipStream_t s);

// Attention (split kernel + merge) of layers 0 .. n_layers - 1 of L, through
// the page tables (paged) or over staged rows.
hipError_t launch_attention_layers(bool paged, const AttnLayers &L, int n_layers, int64_t pt_stride, int max_ctx,
                                   int batch, int budget_blocks, int budget_tokens, float sm_scale, int tps,
                                   hipStream_t s);

// Several queries per sequence (multiscore.hip); n_queries in {4, 8, 16, 32, 64}.
hipError_t launch_multi_score(int n_queries, const uint8_t *keys, const uint16_t *scales, const uint16_t *q_idx,
                              const float *w_idx, const int32_t *q_pos, const int32_t *ctx_len, const int64_t *row0,
                              int64_t n_rows, int batch, int max_ctx, float *out, int64_t bs_stride, hipStream_t s);

// Hot row cache in front of a pinned-host pool (hotcache.hip).
constexpr int kMaxHot = 16384;                   // cache rows per sequence and layer

hipError_t launch_hot_update(const int32_t *sel, const int32_t *n_tok, int batch, int budget_blocks,
                             int budget_tokens, int max_ctx, int32_t *map, int64_t map_stride, int32_t *owner, int H,
                             int2 *fetch, int32_t *n_fetch, int32_t *n_miss_out, hipStream_t s);
hipError_t launch_hot_fetch(const int2 *fetch, const int32_t *n_fetch, int batch, int budget_tokens,
                            const int32_t *pt, int64_t pt_stride, int64_t n_slots, int max_ctx, const void *pool,
                            void *rows, int H, uint32_t *flags, hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);

// Per-layer pointers of the append step, passed by value.
constexpr int kMaxAppendLayers = 64;
struct AppendLayers {
    const float *new_key[kMaxAppendLayers];     // [B][kIdxD]
    const uint8_t *new_row[kMaxAppendLayers];   // [B][kRowBytes]
    uint8_t *keys[kMaxAppendLayers];            // [rows][kIdxD]
    uint16_t *scales[kMaxAppendLayers];         // [rows]
    uint8_t *pool[kMaxAppendLayers];            // [n_slots][kRowBytes]
};

hipError_t launch_append(const AppendLayers &ly, int n_layers, int batch, const int32_t *ctx_len,
                         const int64_t *row0, int64_t n_rows, int64_t pt_stride, int64_t n_slots,
                         const int32_t *new_slot, int32_t *page_table, int32_t *ctx_out, const uint32_t *new_gen,
                         uint32_t *tok_gen, hipStream_t s);
hipError_t launch_move(const AppendLayers &ly, int n_layers, int batch, const int64_t *token, const int32_t *to_slot,
                       const uint32_t *to_gen, int32_t *pt, int64_t pt_stride, int64_t n_slots, uint32_t *tok_gen,
                       hipStream_t s);
hipError_t launch_check_gen(const int32_t *ctx_len, int batch, int64_t pt_stride, const int32_t *pt,
                            const uint32_t *tok_gen, const uint32_t *slot_gen, int64_t n_slots, int32_t *stale,
                            hipStream_t s);

} // namespace qsa
