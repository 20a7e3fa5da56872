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
// Each sequence's histogram is kept in kHistReps copies; scoring workgroup x
// adds into copy x % kHistReps, so that no more than 1/kHistReps of a
// sequence's workgroups queue up on the same counter. Readers sum the copies.
constexpr int kHistReps = 2;

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

// Per-layer pieces of the caller's workspace, carved on the host.
constexpr int kSliceBlocks = 2048;             // blocks per selection slice (one collect workgroup)

struct SelectWs {
    uint32_t *hist;        // [B][kHistReps][kHistBins], zeroed before scoring
    uint32_t *slot_count;  // [B][n_slices][2] per-slice list lengths (definite, candidates)
    int32_t *slot_def;     // [B][n_slices][kSliceBlocks] blocks above the threshold bin
    uint64_t *slot_cand;   // [B][n_slices][kSliceBlocks] blocks inside the threshold bin
    uint64_t *spill;       // [B][spill_stride] candidates past the finish kernel's LDS
    int64_t spill_stride;
    uint32_t *flags;       // the call's flags word (QSA_FLAG_*), or null
    // The index rows of the batch (qsa_decode_step): a sequence whose rows
    // [row0[b], row0[b] + L) fall outside [0, n_rows) was scored as empty, and
    // the selection takes it as empty too. Null when there is no index.
    const int64_t *row0;
    int64_t n_rows;
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
    uint32_t *hist[N];                    // [B][kHistReps][kHistBins] or null
    uint32_t *flags;                      // the call's flags word, or null
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

// Kernel launchers (one translation unit each).
hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s);
hipError_t launch_copy_u32(const uint32_t *src, uint32_t *dst, int64_t n, hipStream_t s);

hipError_t launch_index_score(const uint8_t *keys, const uint16_t *scales, const uint16_t *q_idx,
                              const float *w_idx, const int32_t *ctx_len, const int64_t *row0, int64_t n_rows,
                              int batch, int max_ctx, float *token_scores, float *block_scores, int64_t bs_stride,
                              uint32_t *hist, int budget_blocks, int sink_blocks, int tail_tokens, uint32_t *flags,
                              hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// Index scoring of layers 0 .. n_layers - 1 of L in one launch (grid z =
// layer); token_scores and hist must be null for all layers or for none.
hipError_t launch_index_score_layers(const ScoreLayers &L, int n_layers, const int32_t *ctx_len, const int64_t *row0,
                                     int64_t n_rows, int batch, int max_ctx, int64_t bs_stride, int budget_blocks,
                                     int sink_blocks, int tail_tokens, hipStream_t s, hipEvent_t ev0 = nullptr,
                                     hipEvent_t ev1 = nullptr);

hipError_t launch_block_hist(const float *block_scores, int64_t bs_stride, const int32_t *ctx_len, int batch,
                             int max_ctx, uint32_t *hist, int budget_blocks, int sink_blocks, int tail_tokens,
                             hipStream_t s);

hipError_t launch_select(const float *block_scores, int64_t bs_stride, const int32_t *ctx_len, int batch,
                         int max_ctx, const SelectWs &ws, int budget_blocks, int sink_blocks, int tail_tokens,
                         int32_t *sel, int32_t *n_sel, int32_t *n_tok, hipStream_t s);

// Selection of layers 0 .. n_layers - 1 of L (n_layers <= kMaxChainLayers).
hipError_t launch_select_layers(const SelectLayers &L, int n_layers, int64_t bs_stride, const int32_t *ctx_len,
                                int batch, int max_ctx, int budget_blocks, int sink_blocks, int tail_tokens,
                                hipStream_t s);

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
