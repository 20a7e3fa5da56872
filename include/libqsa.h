/*
 * libqsa.h -- C ABI of libqsa, the QSA sparse-attention decode step for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (sources: the article "双卡RTX4090跑通Qwen3-Next：8并发满血长上下文实测",
 * intro and memory-ledger section; the digest "Оффлоадинг KV-кэша
 * Qwen3.8-Flash-Next в RAM через vLLM", lead paragraph and mechanism /
 * efficiency sections): in every QSA layer of a decode step, each sequence
 *   1. scores every cached token with a compact GPU-resident index key
 *      (66 bytes per token per layer: 64 fp8 e4m3 codes + one fp16 scale),
 *      s_t = sum_h w_h * ReLU(sigma_t * (q_idx_h . k_t));
 *   2. reduces the scores to C4 blocks of 4 adjacent tokens (block score =
 *      max over its valid tokens);
 *   3. keeps at most indexer_budget tokens: the forced blocks (attention sink
 *      at the start, tail ring at the end) plus the best remaining blocks by
 *      (score desc, block index asc);
 *   4. reads only those KV rows (2048 bytes per token per layer) through a
 *      logical-token -> physical-slot page table, from HBM or from pinned host
 *      memory over PCIe;
 *   5. runs GQA softmax attention of the decode query over the gathered rows
 *      (split over tokens, partial results merged by log-sum-exp).
 *
 * Conventions shared by every call
 *   - All pointers are device pointers unless stated otherwise; "host-pinned"
 *     pointers are host allocations made with hipHostMalloc (or torch
 *     pin_memory), read by the GPU directly over PCIe.
 *   - The caller owns every buffer, including the workspace, and every HIP
 *     object the calls use (streams, and the event set of the overlapped
 *     schedules, qsa_step_events_create). The library never allocates, frees,
 *     creates HIP objects or synchronises inside the calls of the decode path;
 *     work is enqueued on the given stream(s) and runs asynchronously. NULL
 *     stream = the default stream. Calls are thread-safe when their
 *     workspaces and event sets differ.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued. Values that live only on the device
 *     (ctx_len, idx_row0, page-table entries, selections) are the caller's
 *     contract. The kernels never read outside the buffers described here:
 *     ctx_len is clamped to [0, max_ctx]; a sequence whose index rows fall
 *     outside [0, n_idx_rows) is treated as empty; a page-table entry outside
 *     [0, n_slots) is read as slot 0 (the result is then unspecified). Calls
 *     that take a workspace report each of these events in a flags word kept
 *     in the workspace (QSA_FLAG_*, read with qsa_read_flags).
 *   - Launch failures return QSA_ERR_HIP; faults surface at the next sync.
 *
 * Data layouts
 *   - Index keys of one layer: idx_keys u8 [rows][idx_dim] (e4m3 codes, OCP
 *     E4M3FN: bias 7, max 448, no infinities) and idx_scales u16 [rows] (IEEE
 *     fp16 bits, sigma_t >= 0), in logical token order; sequence b occupies
 *     rows [idx_row0[b], idx_row0[b] + ctx_len[b]). 66 bytes per token.
 *     The pages give the index row's size only (66 bytes per token per
 *     layer: 64 fp8 codes and one fp16 scale). This library takes the row as
 *     two arrays, codes then scales, rather than one packed 66-byte record:
 *     the same bytes, but every 64-lane load of codes is an aligned, fully
 *     used 1 KB piece, where packed rows would leave 2-byte tails on every
 *     row. The article's memory-ledger section says the index, its
 *     quantisation scales and the page layout were re-aligned against each
 *     other, which this split follows.
 *   - KV pool of one layer: [n_slots][row_bytes], row_bytes = 2 * n_kv_heads *
 *     head_dim * 2 = 2048; a row holds K of KV head 0..n_kv-1, then V of KV
 *     head 0..n_kv-1, each head_dim bf16 values.
 *   - Page table: i32 [batch][pt_stride]; entry [b][t] is the physical slot of
 *     logical token t of sequence b.
 *   - Block selections: i32 [batch][K], K = budget_tokens / block_tokens,
 *     ascending block indices, padded with -1 after n_sel[b] entries.
 *   - Staged rows: [batch][budget_tokens][row_bytes]; row p of sequence b is
 *     the p-th selected token in ascending logical order.
 *   - Queries: q_idx bf16 [batch][idx_heads][idx_dim], w_idx f32
 *     [batch][idx_heads], q bf16 [batch][n_q_heads][head_dim]; outputs f32
 *     [batch][n_q_heads][head_dim]. Query head h reads KV head
 *     h / (n_q_heads / n_kv_heads).
 *
 * Compiled geometry: n_q_heads 16, n_kv_heads 2, head_dim 256, idx_heads 4,
 * idx_dim 64, block_tokens 4. Other values give QSA_ERR_UNSUPPORTED.
 */
#ifndef LIBQSA_H
#define LIBQSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *qsa_stream_t; /* a hipStream_t */

typedef enum {
    QSA_OK = 0,
    QSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misalignment */
    QSA_ERR_UNSUPPORTED = 2,        /* geometry other than the compiled one */
    QSA_ERR_WORKSPACE_TOO_SMALL = 3,
    QSA_ERR_HIP = 4,                /* a HIP launch or runtime call failed */
    QSA_ERR_OUT_OF_SLOTS = 5,       /* a slot pool has no free slot left */
    /* not a status: keeps the type 32 bits wide with every int32 value in its
     * range, so that a value from outside the list (a caller's bug, or another
     * language's integer) is well defined and reported as unknown */
    QSA_STATUS_RANGE_ = 0x7FFFFFFF
} qsa_status_t;

typedef enum {
    QSA_KV_DEVICE = 0,       /* KV pools in device memory (HBM) */
    QSA_KV_HOST_PINNED = 1,  /* KV pools in pinned host memory, read over PCIe */
    /* not a location: every int32 value is in the type's range, so that an
     * unknown value is rejected with QSA_ERR_INVALID_ARGUMENT, not undefined */
    QSA_KV_LOCATION_RANGE_ = 0x7FFFFFFF
} qsa_kv_location_t;

typedef struct {
    int32_t n_q_heads;     /* 16 */
    int32_t n_kv_heads;    /* 2 */
    int32_t head_dim;      /* 256 */
    int32_t idx_heads;     /* 4 indexer heads */
    int32_t idx_dim;       /* 64 (index key = idx_dim e4m3 codes + a fp16 scale) */
    int32_t block_tokens;  /* 4: C4 blocks */
    int32_t budget_tokens; /* indexer_budget, a multiple of block_tokens, <= 8192 */
    int32_t sink_blocks;   /* leading blocks always selected (>= 0) */
    int32_t tail_tokens;   /* blocks holding the last tail_tokens tokens are always selected */
    float sm_scale;        /* softmax scale, normally 1/sqrt(head_dim) */
} qsa_config_t;

typedef struct {
    int32_t batch;             /* B >= 1 (host) */
    int32_t max_ctx;           /* host-side upper bound of ctx_len[b], <= 2^21 */
    const int32_t *ctx_len;    /* device [B] tokens cached per sequence (current one included) */
    const int64_t *idx_row0;   /* device [B] first index row of each sequence */
    const int32_t *page_table; /* device [B][pt_stride] logical token -> slot */
    int64_t pt_stride;         /* >= max_ctx */
    int64_t n_slots;           /* rows in each layer's KV pool */
    int64_t n_idx_rows;        /* rows in each layer's index buffers; a sequence whose rows
                                  [idx_row0, idx_row0 + ctx_len) fall outside is scored as empty */
} qsa_batch_t;

/* Step 1 + 2 (indexer scoring and C4 reduce).
 *   idx_keys     u8  [rows][idx_dim], 16-byte aligned (the 64 codes of each
 *                66-byte index row; the layout note above says why the row's
 *                two parts come as two arrays)
 *   idx_scales   u16 [rows] fp16 bits (the row's last 2 bytes)
 *   q_idx        bf16 bits [B][idx_heads][idx_dim], 16-byte aligned;
 *   w_idx        f32 [B][idx_heads]
 *   token_scores f32 [rows] (same row index as the keys) or NULL
 *   block_scores f32 [B][bs_stride], bs_stride >= ceil(max_ctx / block_tokens);
 *                entries past ceil(ctx_len[b] / block_tokens) are not written. */
qsa_status_t qsa_index_score(const qsa_config_t *cfg, const qsa_batch_t *batch, const uint8_t *idx_keys,
                             const uint16_t *idx_scales, const uint16_t *q_idx, const float *w_idx,
                             float *token_scores, float *block_scores, int64_t bs_stride, qsa_stream_t stream);

/* Step 3 (budgeted block selection), on the given block scores.
 *   sel_blocks i32 [B][K] ascending, -1 padded;  n_sel i32 [B];
 *   n_tok      i32 [B] tokens covered by the selection, or NULL.
 * Exact: the same selection as a full sort by (score desc, index asc); -0.0
 * and +0.0 compare equal, +-inf are ordinary values; NaN scores have no
 * defined rank (the selection stays in bounds, its choice among them is
 * unspecified). Needs qsa_workspace_size(cfg, B, max_ctx, 1, QSA_KV_DEVICE)
 * bytes of workspace (any content; 256-byte aligned). QSA_ERR_INVALID_ARGUMENT
 * if the forced blocks could exceed the budget. */
qsa_status_t qsa_topk_blocks(const qsa_config_t *cfg, const qsa_batch_t *batch, const float *block_scores,
                             int64_t bs_stride, int32_t *sel_blocks, int32_t *n_sel, int32_t *n_tok,
                             void *workspace, size_t workspace_bytes, qsa_stream_t stream);

/* Step 1 for several queries per sequence (prefill or chunked decode): each
 * of the n_queries queries of sequence b scores the index with the same
 * formula, causally -- query i sees tokens t <= q_pos[b][i] -- and gets C4
 * block scores: the max over the block's visible tokens, -inf for a block it
 * does not see. Dense [4 Q x 64] x [64 x L] contraction on the matrix cores.
 *   q_idx bf16 [B][Q][idx_heads][idx_dim] and w_idx f32 [B][Q][idx_heads],
 *   both 16-byte aligned; q_pos int32 [B][Q]; block_scores f32
 *   [B][Q][bs_stride], written for
 *   blocks j < ceil(ctx_len[b] / 4). n_queries in {4, 8, 16, 32, 64}.
 * Each (b, i) row can go to qsa_topk_blocks as a sequence of its own with
 * length q_pos[b][i] + 1. */
qsa_status_t qsa_index_score_multi(const qsa_config_t *cfg, const qsa_batch_t *batch, int32_t n_queries,
                                   const uint8_t *idx_keys, const uint16_t *idx_scales, const uint16_t *q_idx,
                                   const float *w_idx, const int32_t *q_pos, float *block_scores, int64_t bs_stride,
                                   qsa_stream_t stream);

/* Step 4 (page-table translate + row gather). Copies the rows of the selected
 * tokens, in ascending logical order, from kv_pool ([n_slots][row_bytes];
 * device memory, or host-pinned memory for QSA_KV_HOST_PINNED) to kv_out
 * ([B][budget_tokens][row_bytes], device). Writes n_tok[b]. Bit-exact copy. */
qsa_status_t qsa_gather_kv(const qsa_config_t *cfg, const qsa_batch_t *batch, const int32_t *sel_blocks,
                           const int32_t *n_sel, const void *kv_pool, qsa_kv_location_t kv_location,
                           void *kv_out, int32_t *n_tok, qsa_stream_t stream);

/* Step 5 (split-K GQA decode attention + log-sum-exp merge) over staged rows.
 *   q   bf16 bits [B][n_q_heads][head_dim], 16-byte aligned;
 *   kv  [B][budget_tokens][row_bytes], 16-byte aligned
 *   n_tok i32 [B] rows used per sequence (0 gives a zero output)
 *   out f32 [B][n_q_heads][head_dim]
 * The tokens are split in 128-token pieces when the call has at least three
 * quarters as many of them as the device has CUs (budget/128 x B x layers >=
 * 3/4 CUs), else in 64-token pieces; the two splittings round differently (within the
 * same tolerance), so results depend in their last bits on the call's batch
 * and layer count and on the device.
 * Workspace: qsa_workspace_size(cfg, B, 0, 1, QSA_KV_DEVICE) bytes. */
qsa_status_t qsa_sparse_decode(const qsa_config_t *cfg, int32_t batch, const uint16_t *q, const void *kv,
                               const int32_t *n_tok, float *out, void *workspace, size_t workspace_bytes,
                               qsa_stream_t stream);

/* One QSA layer's inputs and outputs for qsa_decode_step. */
/* A hot row cache in HBM in front of a KV pool in pinned host memory
 * (article, memory-ledger section: the full history stays in pinned host
 * memory, the GPU keeps the hot rows, and missing rows are brought back on
 * demand through a per-layer mapping of logical tokens to cache slots).
 * One per layer. Sequence b owns cache rows b*hot_slots .. +hot_slots-1.
 * In every decode step, after the selection:
 *   - selected tokens already in the cache (hits) keep their rows;
 *   - the others (misses), in ascending token order, take the rows that no
 *     hit uses this step, in ascending row order, and unmap each row's
 *     previous token;
 *   - only the misses' rows are read from the host pool (over PCIe);
 *   - attention reads every selected row from the cache.
 * The result is identical to the uncached path's. Initialise map and owner
 * with qsa_hot_reset. hot_slots >= budget_tokens and <= 16384. */
typedef struct qsa_hot_cache {
    void *rows;             /* device [batch][hot_slots][row_bytes] */
    int32_t *map;           /* device [batch][pt_stride]: cache row id of each logical token, or -1 */
    int32_t *owner;         /* device [batch][hot_slots]: logical token held by each row, or -1 */
    int32_t hot_slots;      /* rows per sequence */
    int32_t *n_miss;        /* optional device [batch]: rows fetched over PCIe in the last step */
} qsa_hot_cache_t;

typedef struct {
    const uint8_t *idx_keys;    /* [rows][idx_dim], 16-byte aligned */
    const uint16_t *idx_scales; /* [rows] */
    const uint16_t *q_idx;      /* [B][idx_heads][idx_dim], 16-byte aligned */
    const float *w_idx;         /* [B][idx_heads] */
    const uint16_t *q;          /* [B][n_q_heads][head_dim], 16-byte aligned */
    const void *kv_pool;        /* [n_slots][row_bytes], device or host-pinned, 16-byte aligned */
    const int32_t *page_table;  /* this layer's table, or NULL for batch->page_table */
    float *out;                 /* [B][n_q_heads][head_dim] */
    int32_t *sel_blocks;        /* optional [B][K] copy of the selection, or NULL */
    int32_t *n_sel;             /* optional [B], or NULL */
    const struct qsa_hot_cache *hot; /* optional hot row cache (pinned-host pools only), or NULL */
    void *score_events[2];      /* optional pair of timing-enabled hipEvent_t that take the begin
                                   and end timestamps of this layer's index-scoring kernel (it is
                                   then launched through hipExtLaunchKernel); NULL to skip. Where
                                   one launch scans a group of layers (side streams, no hot
                                   cache), the group's first layer's events time that launch
                                   and the other layers' events are not recorded */
} qsa_layer_t;

/* The whole decode step over n_layers independent QSA layers: for each layer,
 * score -> select -> gather/attend -> merge. With KV in HBM the gather is
 * fused into attention (rows are read through the page table in place). With
 * QSA_KV_HOST_PINNED the selected rows are copied over PCIe into a staging
 * area in the workspace, one buffer per layer (B x budget_tokens x 2048 B).
 * Streams: `side` holds n_side extra streams (all distinct from `compute`);
 * with n_side = 0 (side may then be NULL) every kernel runs in order on
 * `compute`. The layers of a call are independent, so kernels cover several
 * layers at once:
 *   - HBM pools: the layers go in groups of up to 16; one launch scans the
 *     whole group's index, then one launch each of the selection and
 *     attention kernels covers the whole group, all on `compute`, with or
 *     without side streams. With more than 16 layers and a side stream, each
 *     group's selection and attention run on side[0] and overlap the next
 *     group's scan. Further side streams are not used;
 *   - host pools with a hot cache: layer l's whole chain (score, select,
 *     cache update, miss fetch, attend, merge) runs on stream
 *     l % (n_side + 1) of {compute, side[0], side[1], ...}, with at most two
 *     index scans at a time (with n_side = 0, layer after layer);
 *   - host pools without a hot cache and n_side = 0: groups of up to 16
 *     layers, each scanned, selected, gathered and attended with one launch
 *     per kernel;
 *   - host pools without a hot cache, with a side stream: a pipeline over
 *     the layers (digest, efficiency section: the copy of a layer's rows
 *     overlaps the next layer's index scoring). `compute` scores and selects the layers;
 *     side[0] gathers the selected rows over PCIe into their staging
 *     buffers as soon as they are selected, back to back;
 *     `compute` attends the layers once the last rows have arrived. The
 *     layers go in groups of 1, 3, 9, ... layers (the last takes the rest),
 *     one launch per group and step, and the gather runs on a few dozen
 *     workgroups, enough for the PCIe reads, so that the scans beside it
 *     keep the other CUs. side[0] waits for each group's selection on the
 *     event set's signal (a stream memory operation), `compute` for the last
 *     gather on one of its events. Further side streams are not used.
 * The call leaves `compute` ordered after all of its work, so a sync on
 * `compute` covers the step. Results are bit-identical for every schedule
 * of a call (the attention's split size is chosen once per call, as for
 * qsa_sparse_decode with B x n_layers).
 * Events: the schedules that order several streams (side streams with host
 * pools, or with more than 16 layers on HBM pools) record and wait on the
 * events of `events`, a set the caller created with qsa_step_events_create
 * on the current device for at least n_layers layers and n_side side
 * streams; the other schedules need none, and `events` may then be NULL.
 * A set serves one call at a time: calls issued one after another on the
 * same streams may share it, calls from different host threads may not.
 * QSA_ERR_INVALID_ARGUMENT when the schedule needs events and `events` is
 * NULL, too small or made on another device. n_side is at most
 * QSA_MAX_SIDE_STREAMS, n_layers at most QSA_MAX_LAYERS.
 * Workspace: qsa_workspace_size(cfg, B, max_ctx, n_layers, kv_location).
 * The workspace's flags word (qsa_read_flags) is cleared at the start of
 * the call and collects the QSA_FLAG_* events of its kernels. */
#define QSA_MAX_SIDE_STREAMS 8
#define QSA_MAX_LAYERS 64
typedef struct qsa_step_events qsa_step_events_t;
qsa_status_t qsa_decode_step(const qsa_config_t *cfg, const qsa_batch_t *batch, const qsa_layer_t *layers,
                             int32_t n_layers, qsa_kv_location_t kv_location, void *workspace,
                             size_t workspace_bytes, qsa_stream_t compute, const qsa_stream_t *side,
                             int32_t n_side, qsa_step_events_t *events);

/* The HIP events and the signal that order the streams of qsa_decode_step's
 * overlapped schedules, created here (outside any hot path) on the current
 * device, for calls of up to max_layers layers and max_side side streams.
 * The signal is 8 bytes of signal memory (hipExtMallocWithFlags with
 * hipMallocSignalMemory), set to 0 here with a stream write on the null
 * stream, which this call then synchronises; each pinned-host pipeline step
 * writes it with values that only grow. Where signal memory cannot be
 * allocated the set keeps none and the pipeline hands over with its events.
 * Not itself thread-safe: one set per host thread that issues overlapped
 * steps. QSA_ERR_HIP if HIP cannot create the events or set the signal
 * (nothing is then kept). */
qsa_status_t qsa_step_events_create(int32_t max_layers, int32_t max_side, qsa_step_events_t **events);
void qsa_step_events_destroy(qsa_step_events_t *events);

/* Flags a call's kernels raise when device-side values break the contract
 * (each such value is clamped so every read stays in bounds, as described
 * under the conventions above). Kept in a 32-bit word in the workspace. */
#define QSA_FLAG_BAD_SLOT 1u       /* a selected token's page-table entry was outside [0, n_slots)
                                      (its row was read from slot 0) */
#define QSA_FLAG_BAD_INDEX_ROWS 2u /* a sequence's index rows fell outside [0, n_idx_rows)
                                      (it was scored as empty) */
#define QSA_FLAG_BAD_CTX_LEN 4u    /* a ctx_len[b] was outside [0, max_ctx] (it was clamped) */
#define QSA_FLAG_BAD_N_TOK 8u      /* qsa_sparse_decode: an n_tok[b] was outside [0, budget_tokens] */

/* Enqueues a copy of the flags word of `workspace` (a workspace passed to
 * qsa_decode_step, qsa_topk_blocks or qsa_sparse_decode; the word covers the
 * last call that used it, once that call has run) to flags_out (device, one
 * uint32), on `stream`. workspace NULL reads the flags word of
 * qsa_decode_step_static's scratch on the current device. */
qsa_status_t qsa_read_flags(const void *workspace, uint32_t *flags_out, qsa_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid allocation): qsa_decode_step with the
 * workspace taken from a static device array of QSA_STATIC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.
 * The call allocates nothing; the caller still passes every input and output
 * (and, for the schedules that need them, the event set). Its workspace need
 * (qsa_workspace_size) must fit the array, else QSA_ERR_WORKSPACE_TOO_SMALL
 * and nothing is enqueued. Every call on a GPU shares that GPU's array:
 * calls that overlap in time on one GPU (several host threads, or streams
 * not ordered after each other) race and give undefined results. The first
 * call on a device looks up that device's copy of the array (with the device
 * current) and keeps its address. Results are bit-identical to
 * qsa_decode_step's. */
#define QSA_STATIC_SCRATCH_BYTES (64u << 20)
qsa_status_t qsa_decode_step_static(const qsa_config_t *cfg, const qsa_batch_t *batch, const qsa_layer_t *layers,
                                    int32_t n_layers, qsa_kv_location_t kv_location, qsa_stream_t compute,
                                    const qsa_stream_t *side, int32_t n_side, qsa_step_events_t *events);

/* Empties a hot cache: map[b][0..pt_stride) and owner[b][0..hot_slots) = -1
 * for every sequence of the batch. */
qsa_status_t qsa_hot_reset(const qsa_batch_t *batch, const qsa_hot_cache_t *hot, qsa_stream_t stream);

/* Step 0 of the next decode step (article, memory-ledger section: the index,
 * its quantisation scales and the page layout are kept aligned; a token's
 * logical address is mapped to the physical cache slot it was given): the
 * token just decoded enters the cache of every QSA layer. For sequence b with
 * t = batch->ctx_len[b] and s = new_slot[b] (a slot the caller allocated):
 *   - layer l's index row idx_row0[b] + t receives new_idx_key[b] quantised
 *     to e4m3 with one fp16 scale: sigma = fp16(amax / 448) and code_i =
 *     e4m3(x_i / sigma), both divisions in binary32, rounding to nearest even,
 *     magnitudes clamped to 448, all codes 0 when sigma is 0;
 *   - layer l's pool row s receives new_kv_row[b] unchanged;
 *   - page_table[b][t] = s, and ctx_len_out[b] = t + 1.
 * A sequence whose t is outside [0, pt_stride), whose index row falls outside
 * [0, n_idx_rows) or whose slot is outside [0, n_slots) is left untouched and
 * gets ctx_len_out[b] = t. The caller keeps room after each sequence's index
 * rows for the tokens it appends. ctx_len_out may be batch->ctx_len (updated
 * in place) or NULL; page_table is the table to update (usually
 * batch->page_table). At most 64 layers per call. */
typedef struct {
    const float *new_idx_key;   /* device f32 [batch][idx_dim]: the new token's index key */
    const void *new_kv_row;     /* device bf16 [batch][row_elems]: its K and V, pool-row layout */
    uint8_t *idx_keys;          /* this layer's index codes [n_idx_rows][idx_dim] */
    uint16_t *idx_scales;       /* this layer's scales [n_idx_rows] */
    void *kv_pool;              /* this layer's pool [n_slots][row_bytes], device or pinned host */
} qsa_append_layer_t;

qsa_status_t qsa_append_token(const qsa_config_t *cfg, const qsa_batch_t *batch, const qsa_append_layer_t *layers,
                              int32_t n_layers, qsa_kv_location_t kv_location, const int32_t *new_slot,
                              int32_t *page_table, int32_t *ctx_len_out, const uint32_t *new_gen,
                              uint32_t *tok_gen, qsa_stream_t stream);
/* (new_gen, tok_gen: optional device [batch] and [batch][pt_stride]; when
 * tok_gen is given, tok_gen[b][t] receives new_gen[b] (0 without new_gen),
 * the generation of the slot the token was placed in.) */

/* ------------------------------------------------------------ slot leases
 * Host-side slot pool for the KV pools (article, memory-ledger section:
 * leases, generation markers and a tail ring buffer let requests end, be
 * cancelled and hand their cache to new requests; afterwards the cache
 * capacity and slots are back at their initial values).
 *   - n physical slots, each with a generation counter starting at 0; free
 *     slots are handed out lowest first;
 *   - a lease (one request) may take a tail ring of R slots when it opens:
 *     token t is placed in ring slot ring[t % R]; when token t >= R arrives,
 *     token t - R leaves the ring for a body slot taken from the pool, and the
 *     caller moves its rows there (qsa_move_tokens) before appending t;
 *     without a ring every token takes a body slot;
 *   - closing a lease returns all its slots and increments their generations.
 * Host memory only; calls on one pool are serialised by a mutex. */
typedef struct qsa_slot_pool qsa_slot_pool_t;

typedef struct {
    int64_t token;              /* the appended token's position in its sequence */
    int32_t slot;               /* its slot */
    uint32_t generation;        /* that slot's generation */
    int64_t spill_token;        /* token leaving the tail ring, or -1 */
    int32_t spill_from;         /* its ring slot (== slot), or -1 */
    int32_t spill_to;           /* the body slot it moves to, or -1 */
    uint32_t spill_generation;  /* that body slot's generation */
} qsa_slot_plan_t;

qsa_status_t qsa_pool_create(int64_t n_slots, qsa_slot_pool_t **pool);
void qsa_pool_destroy(qsa_slot_pool_t *pool);
/* QSA_ERR_OUT_OF_SLOTS when fewer than ring_slots slots are free. */
qsa_status_t qsa_pool_open(qsa_slot_pool_t *pool, int32_t ring_slots, int32_t *lease);
/* The next token of a lease; QSA_ERR_OUT_OF_SLOTS when a body slot is needed
 * and none is free (the lease is then unchanged). */
qsa_status_t qsa_pool_next(qsa_slot_pool_t *pool, int32_t lease, qsa_slot_plan_t *plan);
qsa_status_t qsa_pool_close(qsa_slot_pool_t *pool, int32_t lease);
int64_t qsa_pool_free_slots(qsa_slot_pool_t *pool);
/* Copies every slot's generation into host gen_out[n_slots]. */
qsa_status_t qsa_pool_generations(qsa_slot_pool_t *pool, uint32_t *gen_out);

/* For each sequence b with token[b] >= 0: every layer's pool row of the
 * token's slot (page_table[b][token[b]]) is copied to slot to_slot[b], the page
 * table points the token there, and tok_gen[b][token[b]] = to_gen[b] when
 * tok_gen is given. Entries out of range leave the sequence untouched.
 * kv_pools: host array of n_layers pool pointers (device or pinned host).
 * token int64 [batch], to_slot int32 [batch], to_gen uint32 [batch] or NULL. */
qsa_status_t qsa_move_tokens(const qsa_batch_t *batch, void *const *kv_pools, int32_t n_layers,
                             qsa_kv_location_t kv_location, const int64_t *token, const int32_t *to_slot,
                             const uint32_t *to_gen, int32_t *page_table, uint32_t *tok_gen, qsa_stream_t stream);

/* stale[b] = number of tokens t < ctx_len[b] whose slot page_table[b][t] is out
 * of range or has a generation slot_gen[slot] other than the one recorded in
 * tok_gen[b][t]. slot_gen: device [n_slots] copy of the pool's generations. */
qsa_status_t qsa_check_generations(const qsa_batch_t *batch, const int32_t *page_table, const uint32_t *tok_gen,
                                   const uint32_t *slot_gen, int32_t *stale, qsa_stream_t stream);

/* Workspace bytes needed by qsa_decode_step (n_layers >= 1); the same call
 * with n_layers = 1 covers qsa_topk_blocks and qsa_sparse_decode. */
size_t qsa_workspace_size(const qsa_config_t *cfg, int32_t batch, int32_t max_ctx, int32_t n_layers,
                          qsa_kv_location_t kv_location);

/* Algorithmic bytes of one layer for one sequence: idx_bytes = ctx * 66
 * (index scan), kv_bytes = n_tok * row_bytes (gathered rows). */
void qsa_layer_bytes(const qsa_config_t *cfg, int64_t ctx, int64_t n_tok, int64_t *idx_bytes, int64_t *kv_bytes);

/* Static description of a status code. */
const char *qsa_status_string(qsa_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* LIBQSA_H */
