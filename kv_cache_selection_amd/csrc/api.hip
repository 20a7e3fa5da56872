// api.hip -- the C ABI of libqsa: host-side validation, workspace carving and
// the per-layer launch sequence of the decode step.
#include <math.h>
#include <atomic>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/libqsa.h"
#include "qsa_internal.h"

using namespace qsa;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int n_split_of(int budget_tokens) { return (budget_tokens + kTPSMin - 1) / kTPSMin; }

// Byte offsets of the workspace pieces. Nothing in it needs clearing but the
// flags word, which the first kernel of each call zeroes.
struct WsLayout {
    int B = 0, K = 0, n_blk_max = 0, n_layers = 0, n_split = 0, budget = 0;
    ListGeom g = {};
    bool lists = false;                             // the selection goes through chunk lists
    size_t flags = 0;
    size_t heads = 0, lists_off = 0, cand = 0, bs = 0, sel = 0, nsel = 0, ntok = 0, po = 0, plse = 0, stage = 0,
           fetch = 0, nfetch = 0;
    size_t per_heads = 0, per_lists = 0, per_cand = 0, per_bs = 0, per_sel = 0, per_nsel = 0, per_ntok = 0,
           per_po = 0, per_plse = 0, per_stage = 0, per_fetch = 0, per_nfetch = 0;
    size_t total = 0;
};

WsLayout make_layout(const qsa_config_t *cfg, int batch, int max_ctx, int n_layers, qsa_kv_location_t loc)
{
    WsLayout w;
    w.B = batch;
    w.K = cfg->budget_tokens / kBT;
    w.budget = cfg->budget_tokens;
    w.n_blk_max = (max_ctx + kBT - 1) / kBT;
    w.n_layers = n_layers;
    w.n_split = n_split_of(cfg->budget_tokens);
    w.g = list_geom(batch, max_ctx, w.K);
    w.lists = uses_lists(max_ctx, w.K);
    const size_t nb = (size_t)(w.n_blk_max > 0 ? w.n_blk_max : 1);
    w.per_heads = w.lists ? align_up((size_t)batch * w.g.n_chunks * 4) : 0;
    w.per_lists = w.lists ? align_up((size_t)batch * w.g.n_chunks * w.g.cap * 8) : 0;
    w.per_cand = w.lists ? align_up((size_t)batch * (nb + (size_t)w.g.n_chunks * w.g.cap) * 8) : 0;
    w.per_bs = align_up((size_t)batch * nb * 4);
    w.per_sel = align_up((size_t)batch * w.K * 4);
    w.per_nsel = align_up((size_t)batch * 4);
    w.per_ntok = align_up((size_t)batch * 4);
    w.per_po = align_up((size_t)batch * kHq * w.n_split * kDh * 4);
    w.per_plse = align_up((size_t)batch * kHq * w.n_split * 4);
    w.per_stage = (loc == QSA_KV_HOST_PINNED) ? align_up((size_t)batch * w.budget * kRowBytes) : 0;
    // hot-cache fetch lists (pinned-host pools only)
    w.per_fetch = (loc == QSA_KV_HOST_PINNED) ? align_up((size_t)batch * w.budget * 8) : 0;
    w.per_nfetch = (loc == QSA_KV_HOST_PINNED) ? align_up((size_t)batch * 4) : 0;
    size_t off = 0;
    w.flags = off;            // one uint32 (QSA_FLAG_*), in its own 256-byte piece
    off += kAlign;
    w.heads = off;
    off += w.per_heads * n_layers;
    w.lists_off = off;
    off += w.per_lists * n_layers;
    w.cand = off;
    off += w.per_cand * n_layers;
    w.bs = off;
    off += w.per_bs * n_layers;
    w.sel = off;
    off += w.per_sel * n_layers;
    w.nsel = off;
    off += w.per_nsel * n_layers;
    w.ntok = off;
    off += w.per_ntok * n_layers;
    w.po = off;
    off += w.per_po * n_layers;
    w.plse = off;
    off += w.per_plse * n_layers;
    w.stage = off;
    off += w.per_stage * (size_t)n_layers;
    w.fetch = off;
    off += w.per_fetch * n_layers;
    w.nfetch = off;
    off += w.per_nfetch * n_layers;
    w.total = off;
    return w;
}

template <typename T> T *at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

SelectWs select_ws(void *ws, const WsLayout &w, int l)
{
    SelectWs s;
    s.heads = w.lists ? at<uint32_t>(ws, w.heads + w.per_heads * l) : nullptr;
    s.lists = w.lists ? at<uint64_t>(ws, w.lists_off + w.per_lists * l) : nullptr;
    s.spill = w.lists ? at<uint64_t>(ws, w.cand + w.per_cand * l) : nullptr;
    s.spill_stride = (w.n_blk_max > 0 ? w.n_blk_max : 1) + (int64_t)w.g.n_chunks * w.g.cap;
    s.flags = at<uint32_t>(ws, w.flags);
    s.row0 = nullptr;
    s.n_rows = 0;
    s.keys = nullptr;
    s.scales = nullptr;
    s.q_idx = nullptr;
    s.w_idx = nullptr;
    return s;
}

// CUs of the current device (read once per device).
int device_cus()
{
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The attention's split size for a call over w.B sequences and w.n_layers
// layers: kTPS tokens when the call's kTPS-token splits number at least
// three quarters of the device's CUs, else kTPSMin. It depends on the call,
// not on how a schedule groups its launches, so that every schedule gives the
// same bits.
AttnWs attn_ws(void *ws, const WsLayout &w, int l)
{
    AttnWs a;
    a.part_o = at<float>(ws, w.po + w.per_po * l);
    a.part_lse = at<float>(ws, w.plse + w.per_plse * l);
    const int64_t big_splits = (int64_t)((w.budget + kTPS - 1) / kTPS) * w.B * w.n_layers;
    a.tps = 4 * big_splits >= 3 * (int64_t)device_cus() ? kTPS : kTPSMin;
    a.n_split = (w.budget + a.tps - 1) / a.tps;
    a.flags = at<uint32_t>(ws, w.flags);
    return a;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

qsa_status_t check_config(const qsa_config_t *c)
{
    if (!c)
        return QSA_ERR_INVALID_ARGUMENT;
    if (c->n_q_heads != kHq || c->n_kv_heads != kHkv || c->head_dim != kDh || c->idx_heads != kIdxH ||
        c->idx_dim != kIdxD || c->block_tokens != kBT)
        return QSA_ERR_UNSUPPORTED;
    if (c->budget_tokens <= 0 || c->budget_tokens % kBT != 0 || c->budget_tokens > kMaxBudget)
        return QSA_ERR_INVALID_ARGUMENT;
    if (c->sink_blocks < 0 || c->tail_tokens < 0 || !isfinite(c->sm_scale))
        return QSA_ERR_INVALID_ARGUMENT;
    // Forced blocks must fit in the budget for every context length.
    const int64_t K = c->budget_tokens / kBT;
    const int64_t tail_blocks = c->tail_tokens > 0 ? ((int64_t)c->tail_tokens + kBT - 1) / kBT + 1 : 0;
    if ((int64_t)c->sink_blocks + tail_blocks > K)
        return QSA_ERR_INVALID_ARGUMENT;
    return QSA_OK;
}

qsa_status_t check_batch(const qsa_batch_t *b, bool need_index, bool need_pt)
{
    if (!b || b->batch < 1 || b->max_ctx < 0 || b->max_ctx > kMaxCtx || !b->ctx_len)
        return QSA_ERR_INVALID_ARGUMENT;
    if (need_index && (!b->idx_row0 || b->n_idx_rows < 0))
        return QSA_ERR_INVALID_ARGUMENT;
    if (need_pt && (!b->page_table || b->pt_stride < b->max_ctx || b->n_slots < 1))
        return QSA_ERR_INVALID_ARGUMENT;
    return QSA_OK;
}

qsa_status_t hip_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_HIP; }

// Address at which the GPU reads a KV pool, or nullptr when it cannot: a pool
// in device memory is used as is; a pool in pinned host memory is translated
// to its device mapping. Pageable or unknown memory is rejected here rather
// than left to fault on the device.
const void *pool_device_ptr(const void *p, qsa_kv_location_t loc)
{
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (loc == QSA_KV_DEVICE)
        return (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) ? p : nullptr;
    if (a.type != hipMemoryTypeHost || !a.devicePointer)
        return nullptr;
    if (a.hostPointer)
        return static_cast<const char *>(a.devicePointer) +
               (static_cast<const char *>(p) - static_cast<const char *>(a.hostPointer));
    return a.devicePointer;
}

// The number of events a schedule of qsa_decode_step records: fork and join
// events plus one or two per layer (the scans of the hot-cache schedule, the
// layer groups of the HBM schedule, the selections and gathers of the
// pinned-host pipeline).
int events_needed(int n_layers, int n_side) { return 3 * n_layers + n_side + 1; }

// Workgroups of the pinned-host pipeline's gathers: 64 x 32 KB of PCIe reads
// in flight keep the link busy (32 did not; more took CUs from the scans
// beside them and the step got slower).
constexpr int kPipeGatherWgs = 64;

} // namespace

// Scratch of qsa_decode_step_static: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends. In host code its name
// is only a stand-in for the symbol: the device address of each GPU's copy is
// fetched once per device with hipGetSymbolAddress, and only that address is
// ever passed to kernels or fills.
static __device__ __align__(256) uint8_t scratch[QSA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, looked up on the first call on
// each device (with that device current); nullptr with *err set on failure.
void *static_scratch(qsa_status_t *err)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = QSA_ERR_HIP;
        return nullptr;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
            (void)hipGetLastError();
            *err = QSA_ERR_HIP;
            return nullptr;
        }
        p = q;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

} // namespace

// The caller's event set (qsa_step_events_create): HIP events, and one signal
// (signal memory, written and waited on by stream memory operations) with the
// last value written to it.
struct qsa_step_events {
    int device;
    int max_layers, max_side;
    std::vector<hipEvent_t> ev;
    uint64_t *signal = nullptr;
    uint64_t epoch = 0;
};

extern "C" {

qsa_status_t qsa_step_events_create(int32_t max_layers, int32_t max_side, qsa_step_events_t **events)
{
    if (!events || max_layers < 1 || max_side < 0 || max_side > QSA_MAX_SIDE_STREAMS)
        return QSA_ERR_INVALID_ARGUMENT;
    *events = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return QSA_ERR_HIP;
    qsa_step_events *e = new (std::nothrow) qsa_step_events;
    if (!e)
        return QSA_ERR_HIP;
    e->device = dev;
    e->max_layers = max_layers;
    e->max_side = max_side;
    const int n = events_needed(max_layers, max_side);
    e->ev.reserve((size_t)n);
    for (int i = 0; i < n; i++) {
        hipEvent_t h;
        if (hipEventCreateWithFlags(&h, hipEventDisableTiming) != hipSuccess) {
            qsa_step_events_destroy(e);
            return QSA_ERR_HIP;
        }
        e->ev.push_back(h);
    }
    // A fresh signal holds 1, so it is set to 0 before its first use; the
    // values written later count up from there. Where signal memory is not
    // available the pipeline hands over with events instead.
    if (hipExtMallocWithFlags((void **)&e->signal, sizeof(uint64_t), hipMallocSignalMemory) != hipSuccess) {
        (void)hipGetLastError();
        e->signal = nullptr;
    } else if (hipStreamWriteValue64(nullptr, e->signal, 0, 0) != hipSuccess ||
               hipStreamSynchronize(nullptr) != hipSuccess) {
        qsa_step_events_destroy(e);
        return QSA_ERR_HIP;
    }
    *events = e;
    return QSA_OK;
}

void qsa_step_events_destroy(qsa_step_events_t *events)
{
    if (!events)
        return;
    for (hipEvent_t h : events->ev)
        (void)hipEventDestroy(h);
    if (events->signal)
        (void)hipFree(events->signal);
    delete events;
}

qsa_status_t qsa_read_flags(const void *workspace, uint32_t *flags_out, qsa_stream_t stream)
{
    if (!flags_out || !aligned(flags_out, 4) || (workspace && !aligned(workspace, kAlign)))
        return QSA_ERR_INVALID_ARGUMENT;
    if (!workspace) {
        qsa_status_t err = QSA_OK;
        if (!(workspace = static_scratch(&err)))
            return err;
    }
    return hip_status(launch_copy_u32(static_cast<const uint32_t *>(workspace), flags_out, 1, (hipStream_t)stream));
}

size_t qsa_workspace_size(const qsa_config_t *cfg, int32_t batch, int32_t max_ctx, int32_t n_layers,
                          qsa_kv_location_t kv_location)
{
    if (check_config(cfg) != QSA_OK || batch < 1 || max_ctx < 0 || max_ctx > kMaxCtx || n_layers < 1)
        return 0;
    return make_layout(cfg, batch, max_ctx, n_layers, kv_location).total;
}

void qsa_layer_bytes(const qsa_config_t *cfg, int64_t ctx, int64_t n_tok, int64_t *idx_bytes, int64_t *kv_bytes)
{
    const int64_t idx_row = cfg ? (int64_t)cfg->idx_dim + 2 : 0;
    const int64_t kv_row = cfg ? 2LL * cfg->n_kv_heads * cfg->head_dim * 2 : 0;
    if (idx_bytes)
        *idx_bytes = ctx * idx_row;
    if (kv_bytes)
        *kv_bytes = n_tok * kv_row;
}

const char *qsa_status_string(qsa_status_t s)
{
    switch (s) {
    case QSA_OK:
        return "ok";
    case QSA_ERR_INVALID_ARGUMENT:
        return "invalid argument";
    case QSA_ERR_UNSUPPORTED:
        return "unsupported geometry";
    case QSA_ERR_WORKSPACE_TOO_SMALL:
        return "workspace too small";
    case QSA_ERR_HIP:
        return "HIP runtime error";
    case QSA_ERR_OUT_OF_SLOTS:
        return "slot pool exhausted";
    default:
        return "unknown status";
    }
}

qsa_status_t qsa_index_score(const qsa_config_t *cfg, const qsa_batch_t *batch, const uint8_t *idx_keys,
                             const uint16_t *idx_scales, const uint16_t *q_idx, const float *w_idx,
                             float *token_scores, float *block_scores, int64_t bs_stride, qsa_stream_t stream)
{
    qsa_status_t st = check_config(cfg);
    if (st != QSA_OK)
        return st;
    if ((st = check_batch(batch, true, false)) != QSA_OK)
        return st;
    if (!idx_keys || !idx_scales || !q_idx || !w_idx || !block_scores || !aligned(idx_keys, 16) ||
        !aligned(idx_scales, 2) || !aligned(q_idx, 16) || !aligned(w_idx, 4) ||
        bs_stride < (batch->max_ctx + kBT - 1) / kBT)
        return QSA_ERR_INVALID_ARGUMENT;
    const ListGeom g = {};
    return hip_status(launch_index_score(idx_keys, idx_scales, q_idx, w_idx, batch->ctx_len, batch->idx_row0,
                                         batch->n_idx_rows, batch->batch, batch->max_ctx, token_scores, block_scores,
                                         bs_stride, nullptr, nullptr, g, 0, 0, 0, nullptr, (hipStream_t)stream));
}

qsa_status_t qsa_index_score_multi(const qsa_config_t *cfg, const qsa_batch_t *batch, int32_t n_queries,
                                   const uint8_t *idx_keys, const uint16_t *idx_scales, const uint16_t *q_idx,
                                   const float *w_idx, const int32_t *q_pos, float *block_scores, int64_t bs_stride,
                                   qsa_stream_t stream)
{
    qsa_status_t st = check_config(cfg);
    if (st != QSA_OK)
        return st;
    if ((st = check_batch(batch, true, false)) != QSA_OK)
        return st;
    if (!(n_queries == 4 || n_queries == 8 || n_queries == 16 || n_queries == 32 || n_queries == 64))
        return QSA_ERR_UNSUPPORTED;
    if (!idx_keys || !idx_scales || !q_idx || !w_idx || !q_pos || !block_scores || !aligned(idx_keys, 16) ||
        !aligned(idx_scales, 2) || !aligned(q_idx, 16) || !aligned(w_idx, 16) || !aligned(q_pos, 4) ||
        bs_stride < (batch->max_ctx + kBT - 1) / kBT)
        return QSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_multi_score(n_queries, idx_keys, idx_scales, q_idx, w_idx, q_pos, batch->ctx_len,
                                         batch->idx_row0, batch->n_idx_rows, batch->batch, batch->max_ctx,
                                         block_scores, bs_stride, (hipStream_t)stream));
}

qsa_status_t qsa_topk_blocks(const qsa_config_t *cfg, const qsa_batch_t *batch, const float *block_scores,
                             int64_t bs_stride, int32_t *sel_blocks, int32_t *n_sel, int32_t *n_tok,
                             void *workspace, size_t workspace_bytes, qsa_stream_t stream)
{
    qsa_status_t st = check_config(cfg);
    if (st != QSA_OK)
        return st;
    if ((st = check_batch(batch, false, false)) != QSA_OK)
        return st;
    if (!block_scores || !sel_blocks || !n_sel || !workspace || !aligned(workspace, kAlign) ||
        bs_stride < (batch->max_ctx + kBT - 1) / kBT)
        return QSA_ERR_INVALID_ARGUMENT;
    const WsLayout w = make_layout(cfg, batch->batch, batch->max_ctx, 1, QSA_KV_DEVICE);
    if (workspace_bytes < w.total)
        return QSA_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t s = (hipStream_t)stream;
    const SelectWs sw = select_ws(workspace, w, 0);
    hipError_t e = launch_zero_u32(at<uint32_t>(workspace, w.flags), 1, s);
    if (e == hipSuccess && w.lists)
        e = launch_list_build(block_scores, bs_stride, batch->ctx_len, batch->batch, batch->max_ctx, sw.heads,
                              sw.lists, w.g, w.K, cfg->sink_blocks, cfg->tail_tokens, s);
    if (e == hipSuccess)
        e = launch_select(block_scores, bs_stride, batch->ctx_len, batch->batch, batch->max_ctx, sw, w.g, w.K,
                          cfg->sink_blocks, cfg->tail_tokens, sel_blocks, n_sel, n_tok, s);
    return hip_status(e);
}

qsa_status_t qsa_gather_kv(const qsa_config_t *cfg, const qsa_batch_t *batch, const int32_t *sel_blocks,
                           const int32_t *n_sel, const void *kv_pool, qsa_kv_location_t kv_location, void *kv_out,
                           int32_t *n_tok, qsa_stream_t stream)
{
    qsa_status_t st = check_config(cfg);
    if (st != QSA_OK)
        return st;
    if ((st = check_batch(batch, false, true)) != QSA_OK)
        return st;
    if (!sel_blocks || !n_sel || !kv_pool || !kv_out || !aligned(kv_pool, 16) || !aligned(kv_out, 16) ||
        (kv_location != QSA_KV_DEVICE && kv_location != QSA_KV_HOST_PINNED))
        return QSA_ERR_INVALID_ARGUMENT;
    const void *pool = pool_device_ptr(kv_pool, kv_location);
    if (!pool)
        return QSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_gather(sel_blocks, n_sel, batch->ctx_len, batch->batch, batch->max_ctx,
                                    batch->page_table, batch->pt_stride, batch->n_slots, pool, kv_out,
                                    cfg->budget_tokens / kBT, cfg->budget_tokens, n_tok, nullptr,
                                    (hipStream_t)stream));
}

qsa_status_t qsa_sparse_decode(const qsa_config_t *cfg, int32_t batch, const uint16_t *q, const void *kv,
                               const int32_t *n_tok, float *out, void *workspace, size_t workspace_bytes,
                               qsa_stream_t stream)
{
    qsa_status_t st = check_config(cfg);
    if (st != QSA_OK)
        return st;
    if (batch < 1 || !q || !kv || !n_tok || !out || !workspace || !aligned(q, 16) || !aligned(kv, 16) ||
        !aligned(n_tok, 4) || !aligned(out, 4) || !aligned(workspace, kAlign))
        return QSA_ERR_INVALID_ARGUMENT;
    const WsLayout w = make_layout(cfg, batch, 0, 1, QSA_KV_DEVICE);
    if (workspace_bytes < w.total)
        return QSA_ERR_WORKSPACE_TOO_SMALL;
    hipError_t e = launch_zero_u32(at<uint32_t>(workspace, w.flags), 1, (hipStream_t)stream);
    if (e == hipSuccess)
        e = launch_attention_staged(q, kv, n_tok, batch, cfg->budget_tokens, cfg->sm_scale, attn_ws(workspace, w, 0),
                                    out, (hipStream_t)stream);
    return hip_status(e);
}

qsa_status_t qsa_hot_reset(const qsa_batch_t *batch, const qsa_hot_cache_t *hot, qsa_stream_t stream)
{
    if (!batch || batch->batch < 1 || batch->pt_stride < 1 || !hot || !hot->map || !hot->owner ||
        hot->hot_slots < 1 || hot->hot_slots > kMaxHot)
        return QSA_ERR_INVALID_ARGUMENT;
    hipError_t e = launch_fill_i32(hot->map, (int64_t)batch->batch * batch->pt_stride, -1, (hipStream_t)stream);
    if (e == hipSuccess)
        e = launch_fill_i32(hot->owner, (int64_t)batch->batch * hot->hot_slots, -1, (hipStream_t)stream);
    return hip_status(e);
}

qsa_status_t qsa_append_token(const qsa_config_t *cfg, const qsa_batch_t *batch, const qsa_append_layer_t *layers,
                              int32_t n_layers, qsa_kv_location_t kv_location, const int32_t *new_slot,
                              int32_t *page_table, int32_t *ctx_len_out, const uint32_t *new_gen,
                              uint32_t *tok_gen, qsa_stream_t stream)
{
    qsa_status_t st = check_config(cfg);
    if (st != QSA_OK)
        return st;
    if (!batch || batch->batch < 1 || !batch->ctx_len || !batch->idx_row0 || batch->n_idx_rows < 0 ||
        batch->pt_stride < 1 || batch->n_slots < 1)
        return QSA_ERR_INVALID_ARGUMENT;
    if (!layers || n_layers < 1 || n_layers > kMaxAppendLayers || !new_slot || !page_table ||
        (kv_location != QSA_KV_DEVICE && kv_location != QSA_KV_HOST_PINNED))
        return QSA_ERR_INVALID_ARGUMENT;
    AppendLayers ly = {};
    for (int l = 0; l < n_layers; l++) {
        const qsa_append_layer_t &L = layers[l];
        if (!L.new_idx_key || !L.new_kv_row || !L.idx_keys || !L.idx_scales || !L.kv_pool ||
            !aligned(L.new_idx_key, 4) || !aligned(L.new_kv_row, 16) || !aligned(L.kv_pool, 16) ||
            !aligned(L.idx_scales, 2))
            return QSA_ERR_INVALID_ARGUMENT;
        const void *pool = pool_device_ptr(L.kv_pool, kv_location);
        if (!pool)
            return QSA_ERR_INVALID_ARGUMENT;
        ly.new_key[l] = L.new_idx_key;
        ly.new_row[l] = static_cast<const uint8_t *>(L.new_kv_row);
        ly.keys[l] = L.idx_keys;
        ly.scales[l] = L.idx_scales;
        ly.pool[l] = static_cast<uint8_t *>(const_cast<void *>(pool));
    }
    return hip_status(launch_append(ly, n_layers, batch->batch, batch->ctx_len, batch->idx_row0, batch->n_idx_rows,
                                    batch->pt_stride, batch->n_slots, new_slot, page_table, ctx_len_out, new_gen,
                                    tok_gen, (hipStream_t)stream));
}

qsa_status_t qsa_move_tokens(const qsa_batch_t *batch, void *const *kv_pools, int32_t n_layers,
                             qsa_kv_location_t kv_location, const int64_t *token, const int32_t *to_slot,
                             const uint32_t *to_gen, int32_t *page_table, uint32_t *tok_gen, qsa_stream_t stream)
{
    if (!batch || batch->batch < 1 || batch->pt_stride < 1 || batch->n_slots < 1 || !kv_pools || n_layers < 1 ||
        n_layers > kMaxAppendLayers || !token || !to_slot || !page_table ||
        (kv_location != QSA_KV_DEVICE && kv_location != QSA_KV_HOST_PINNED))
        return QSA_ERR_INVALID_ARGUMENT;
    AppendLayers ly = {};
    for (int l = 0; l < n_layers; l++) {
        if (!kv_pools[l] || !aligned(kv_pools[l], 16))
            return QSA_ERR_INVALID_ARGUMENT;
        const void *pool = pool_device_ptr(kv_pools[l], kv_location);
        if (!pool)
            return QSA_ERR_INVALID_ARGUMENT;
        ly.pool[l] = static_cast<uint8_t *>(const_cast<void *>(pool));
    }
    return hip_status(launch_move(ly, n_layers, batch->batch, token, to_slot, to_gen, page_table, batch->pt_stride,
                                  batch->n_slots, tok_gen, (hipStream_t)stream));
}

qsa_status_t qsa_check_generations(const qsa_batch_t *batch, const int32_t *page_table, const uint32_t *tok_gen,
                                   const uint32_t *slot_gen, int32_t *stale, qsa_stream_t stream)
{
    if (!batch || batch->batch < 1 || !batch->ctx_len || batch->pt_stride < 1 || batch->n_slots < 1 ||
        !page_table || !tok_gen || !slot_gen || !stale)
        return QSA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_check_gen(batch->ctx_len, batch->batch, batch->pt_stride, page_table, tok_gen, slot_gen,
                                       batch->n_slots, stale, (hipStream_t)stream));
}

qsa_status_t qsa_decode_step(const qsa_config_t *cfg, const qsa_batch_t *batch, const qsa_layer_t *layers,
                             int32_t n_layers, qsa_kv_location_t kv_location, void *workspace,
                             size_t workspace_bytes, qsa_stream_t compute, const qsa_stream_t *side,
                             int32_t n_side, qsa_step_events_t *events)
{
    qsa_status_t st = check_config(cfg);
    if (st != QSA_OK)
        return st;
    if ((st = check_batch(batch, true, true)) != QSA_OK)
        return st;
    if (!layers || n_layers < 1 || n_layers > QSA_MAX_LAYERS || !workspace || !aligned(workspace, kAlign) ||
        (kv_location != QSA_KV_DEVICE && kv_location != QSA_KV_HOST_PINNED))
        return QSA_ERR_INVALID_ARGUMENT;
    int n_hot = 0;
    for (int l = 0; l < n_layers; l++) {
        const qsa_layer_t &L = layers[l];
        if (!L.idx_keys || !L.idx_scales || !L.q_idx || !L.w_idx || !L.q || !L.kv_pool || !L.out ||
            !aligned(L.idx_keys, 16) || !aligned(L.idx_scales, 2) || !aligned(L.q_idx, 16) || !aligned(L.w_idx, 4) ||
            !aligned(L.q, 16) || !aligned(L.kv_pool, 16) || !aligned(L.out, 4) ||
            (L.page_table && !aligned(L.page_table, 4)))
            return QSA_ERR_INVALID_ARGUMENT;
        if (L.hot) {
            const qsa_hot_cache_t &H = *L.hot;
            if (kv_location != QSA_KV_HOST_PINNED || !H.rows || !H.map || !H.owner || !aligned(H.rows, 16) ||
                H.hot_slots < cfg->budget_tokens || H.hot_slots > kMaxHot ||
                (int64_t)batch->batch * H.hot_slots > INT32_MAX)
                return QSA_ERR_INVALID_ARGUMENT;
            n_hot++;
        }
    }
    if (n_hot != 0 && n_hot != n_layers)
        return QSA_ERR_INVALID_ARGUMENT;            // every layer cached, or none
    const bool hot = n_hot > 0;
    if (n_side < 0 || n_side > QSA_MAX_SIDE_STREAMS || (n_side > 0 && !side))
        return QSA_ERR_INVALID_ARGUMENT;
    for (int k = 0; k < n_side; k++) {
        if (side[k] == compute)
            return QSA_ERR_INVALID_ARGUMENT;
        for (int k2 = 0; k2 < k; k2++)
            if (side[k] == side[k2])
                return QSA_ERR_INVALID_ARGUMENT;
    }
    // The schedules that order several streams take their events from the
    // caller's set: the hot-cache schedule, the pinned-host pipeline, and HBM
    // pools with more layers than one group. Side streams that a schedule
    // does not use are ignored.
    const bool offload = kv_location == QSA_KV_HOST_PINNED;
    const bool two_streams = n_side > 0;
    const int NS = (offload && !hot) ? (n_side > 0 ? 1 : 0) : n_side;
    const bool needs_events = two_streams && (hot || offload || n_layers > kMaxChainLayers);
    const hipEvent_t *ev = nullptr;
    if (needs_events) {
        if (!events || events->max_layers < n_layers || events->max_side < NS ||
            (int)events->ev.size() < events_needed(n_layers, NS))
            return QSA_ERR_INVALID_ARGUMENT;
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return QSA_ERR_HIP;
        if (events->device != dev)
            return QSA_ERR_INVALID_ARGUMENT;
        ev = events->ev.data();
    }
    const WsLayout w = make_layout(cfg, batch->batch, batch->max_ctx, n_layers, kv_location);
    if (workspace_bytes < w.total)
        return QSA_ERR_WORKSPACE_TOO_SMALL;
    const void *pools[QSA_MAX_LAYERS];
    for (int l = 0; l < n_layers; l++) {
        pools[l] = pool_device_ptr(layers[l].kv_pool, kv_location);
        if (!pools[l])
            return QSA_ERR_INVALID_ARGUMENT;
    }

    hipStream_t sc = (hipStream_t)compute;
    const int B = batch->batch;
    const int K = w.K;
    const int64_t bs_stride = w.n_blk_max > 0 ? w.n_blk_max : 1;

    // Per-layer pieces.
    struct Lw {
        const int32_t *pt;
        float *bs;
        int32_t *sel, *nsel, *ntok;
        SelectWs sw;
        AttnWs aw;
        void *stage;
        int2 *fetch;
        int32_t *nfetch;
    };
    Lw lw[QSA_MAX_LAYERS];
    for (int l = 0; l < n_layers; l++) {
        const qsa_layer_t &Ly = layers[l];
        Lw &x = lw[l];
        x.pt = Ly.page_table ? Ly.page_table : batch->page_table;
        x.bs = at<float>(workspace, w.bs + w.per_bs * l);
        x.sel = Ly.sel_blocks ? Ly.sel_blocks : at<int32_t>(workspace, w.sel + w.per_sel * l);
        x.nsel = Ly.n_sel ? Ly.n_sel : at<int32_t>(workspace, w.nsel + w.per_nsel * l);
        x.ntok = at<int32_t>(workspace, w.ntok + w.per_ntok * l);
        x.sw = select_ws(workspace, w, l);
        x.sw.row0 = batch->idx_row0;
        x.sw.n_rows = batch->n_idx_rows;
        // the scans keep few block scores; the selection scores again what it re-reads
        x.sw.keys = Ly.idx_keys;
        x.sw.scales = Ly.idx_scales;
        x.sw.q_idx = Ly.q_idx;
        x.sw.w_idx = Ly.w_idx;
        x.aw = attn_ws(workspace, w, l);
        x.stage = offload ? at<void>(workspace, w.stage + w.per_stage * l) : nullptr;
        x.fetch = offload ? at<int2>(workspace, w.fetch + w.per_fetch * l) : nullptr;
        x.nfetch = offload ? at<int32_t>(workspace, w.nfetch + w.per_nfetch * l) : nullptr;
    }
    uint32_t *const flags = at<uint32_t>(workspace, w.flags);
    // The first scan of the call clears the flags word (and raises none
    // itself), unless a fill kernel has done so before it.
    bool flags_cleared = false;
    auto score = [&](int l, hipStream_t s) {
        const qsa_layer_t &Ly = layers[l];
        uint32_t *clear = flags_cleared ? nullptr : flags;
        flags_cleared = true;
        return launch_index_score(Ly.idx_keys, Ly.idx_scales, Ly.q_idx, Ly.w_idx, batch->ctx_len, batch->idx_row0,
                                  batch->n_idx_rows, B, batch->max_ctx, nullptr, lw[l].bs, bs_stride, lw[l].sw.heads,
                                  lw[l].sw.lists, w.g, K, cfg->sink_blocks, cfg->tail_tokens,
                                  clear ? nullptr : flags, s, (hipEvent_t)Ly.score_events[0],
                                  (hipEvent_t)Ly.score_events[1], clear, true);
    };
    auto select = [&](int l, hipStream_t s) {
        return launch_select(lw[l].bs, bs_stride, batch->ctx_len, B, batch->max_ctx, lw[l].sw, w.g, K,
                             cfg->sink_blocks, cfg->tail_tokens, lw[l].sel, lw[l].nsel, lw[l].ntok, s);
    };
    // Hot cache: update the mapping, fetch the misses over PCIe, then attend
    // the cached rows with the mapping as the page table.
    auto attend_hot = [&](int l, hipStream_t s) {
        const qsa_hot_cache_t &H = *layers[l].hot;
        hipError_t r = launch_hot_update(lw[l].sel, lw[l].ntok, B, K, cfg->budget_tokens, batch->max_ctx, H.map,
                                         batch->pt_stride, H.owner, H.hot_slots, lw[l].fetch, lw[l].nfetch, H.n_miss,
                                         s);
        if (r == hipSuccess)
            r = launch_hot_fetch(lw[l].fetch, lw[l].nfetch, B, cfg->budget_tokens, lw[l].pt, batch->pt_stride,
                                 batch->n_slots, batch->max_ctx, pools[l], H.rows, H.hot_slots, flags, s);
        if (r == hipSuccess)
            r = launch_attention_paged(layers[l].q, H.rows, H.map, batch->pt_stride, (int64_t)B * H.hot_slots,
                                       lw[l].sel, lw[l].ntok, batch->ctx_len, batch->max_ctx, B, K,
                                       cfg->budget_tokens, cfg->sm_scale, lw[l].aw, layers[l].out, s);
        return r;
    };
    auto attend_paged = [&](int l, hipStream_t s) {
        if (hot)
            return attend_hot(l, s);
        return launch_attention_paged(layers[l].q, pools[l], lw[l].pt, batch->pt_stride, batch->n_slots, lw[l].sel,
                                      lw[l].ntok, batch->ctx_len, batch->max_ctx, B, K, cfg->budget_tokens,
                                      cfg->sm_scale, lw[l].aw, layers[l].out, s);
    };
    auto gather = [&](int l, hipStream_t s) {
        return launch_gather(lw[l].sel, lw[l].nsel, batch->ctx_len, B, batch->max_ctx, lw[l].pt, batch->pt_stride,
                             batch->n_slots, pools[l], lw[l].stage, K, cfg->budget_tokens, lw[l].ntok, flags, s);
    };
    auto attend_staged = [&](int l, hipStream_t s) {
        return launch_attention_staged(layers[l].q, lw[l].stage, lw[l].ntok, B, cfg->budget_tokens, cfg->sm_scale,
                                       lw[l].aw, layers[l].out, s);
    };

    hipError_t e = hipSuccess;
    if (two_streams && hot) {
        // This schedule starts scans on several streams from an event after
        // the clear, so the clear is a kernel of its own. (The pinned-host
        // pipeline starts its side stream after the first group's selection,
        // so its first scan clears the word.)
        e = launch_zero_u32(flags, 1, sc);
        flags_cleared = true;
    }

    if (!two_streams && hot) {
        // Hot cache, one stream: every layer's kernels in order (its cache
        // update and miss fetch sit between its selection and attention).
        for (int l = 0; l < n_layers && e == hipSuccess; l++) {
            e = score(l, sc);
            if (e == hipSuccess)
                e = select(l, sc);
            if (e == hipSuccess && (!offload || hot))
                e = attend_paged(l, sc);
            if (e == hipSuccess && offload && !hot)
                e = gather(l, sc);
            if (e == hipSuccess && offload && !hot)
                e = attend_staged(l, sc);
        }
        return hip_status(e);
    }

    // The per-layer pointer tables of layers l0 .. l0 + nl - 1 (HBM pools).
    auto hbm_tables = [&](int l0, int nl, ScoreLayers &CL, SelectLayers &SL, AttnLayers &AL) {
        CL.flags = l0 == 0 ? nullptr : flags;      // the first scan clears the word instead
        CL.drop_listed_bs = 1;
        AL.flags = flags;
        for (int i = 0; i < nl; i++) {
            const int l = l0 + i;
            const qsa_layer_t &Ly = layers[l];
            CL.keys[i] = Ly.idx_keys;
            CL.scales[i] = Ly.idx_scales;
            CL.q_idx[i] = Ly.q_idx;
            CL.w_idx[i] = Ly.w_idx;
            CL.block_scores[i] = lw[l].bs;
            CL.heads[i] = lw[l].sw.heads;
            CL.lists[i] = lw[l].sw.lists;
            SL.bs[i] = lw[l].bs;
            SL.ws[i] = lw[l].sw;
            SL.sel[i] = lw[l].sel;
            SL.n_sel[i] = lw[l].nsel;
            SL.n_tok[i] = lw[l].ntok;
            AL.q[i] = Ly.q;
            AL.rows[i] = static_cast<const uint8_t *>(pools[l]);
            AL.pt[i] = lw[l].pt;
            AL.n_slots[i] = batch->n_slots;
            AL.sel[i] = lw[l].sel;
            AL.n_tok[i] = lw[l].ntok;
            AL.part_o[i] = lw[l].aw.part_o;
            AL.part_lse[i] = lw[l].aw.part_lse;
            AL.out[i] = Ly.out;
        }
    };

    if (!offload && !hot) {
        // Pools in HBM. The layers go in groups of up to kMaxChainLayers: one
        // launch scans the whole group's index (the layer is a grid
        // coordinate, so the scan streams without a break between layers),
        // then one launch each of the selection, attention and merge kernels
        // covers the whole group. A group costs one latency chain instead of
        // one per layer, and its attention is a single wide launch; running
        // the chains during the scans instead only takes CUs and bandwidth
        // from the scans, and every dependency between streams adds 6-13 us
        // before the waiting kernel starts. With one group everything runs
        // on the compute stream, with or without side streams. With several
        // and a side stream, the chains run on side 0, so a group's chain
        // overlaps the next group's scan. The first layer's score events of a
        // group time that group's scan.
        const hipStream_t cs = two_streams && n_layers > kMaxChainLayers ? (hipStream_t)side[0] : sc;
        const int n_used = cs != sc ? 1 : 0;
        if (e == hipSuccess && n_used) {
            e = hipEventRecord(ev[0], sc);
            if (e == hipSuccess)
                e = hipStreamWaitEvent(cs, ev[0], 0);
        }
        for (int l0 = 0; l0 < n_layers && e == hipSuccess; l0 += kMaxChainLayers) {
            const int nl = n_layers - l0 < kMaxChainLayers ? n_layers - l0 : kMaxChainLayers;
            ScoreLayers CL = {};
            SelectLayers SL = {};
            AttnLayers AL = {};
            hbm_tables(l0, nl, CL, SL, AL);
            e = launch_index_score_layers(CL, nl, batch->ctx_len, batch->idx_row0, batch->n_idx_rows, B,
                                          batch->max_ctx, bs_stride, w.g, K, cfg->sink_blocks, cfg->tail_tokens, sc,
                                          (hipEvent_t)layers[l0].score_events[0],
                                          (hipEvent_t)layers[l0].score_events[1], l0 == 0 ? flags : nullptr);
            if (e == hipSuccess && cs != sc) {
                e = hipEventRecord(ev[1 + NS + l0], sc);
                if (e == hipSuccess)
                    e = hipStreamWaitEvent(cs, ev[1 + NS + l0], 0);
            }
            if (e == hipSuccess)
                e = launch_select_layers(SL, nl, bs_stride, batch->ctx_len, B, batch->max_ctx, w.g, K,
                                         cfg->sink_blocks, cfg->tail_tokens, cs);
            if (e == hipSuccess)
                e = launch_attention_layers(true, AL, nl, batch->pt_stride, batch->max_ctx, B, K,
                                            cfg->budget_tokens, cfg->sm_scale, lw[l0].aw.tps, cs);
        }
        // The caller synchronises on the compute stream: join the side stream.
        if (e == hipSuccess && n_used) {
            e = hipEventRecord(ev[1], cs);
            if (e == hipSuccess)
                e = hipStreamWaitEvent(sc, ev[1], 0);
        }
        return hip_status(e);
    }

    if (hot) {
        // Hot-cached pinned-host pools: layer l's whole chain (score, select,
        // hot-cache update and fetch, attend, merge) runs on stream
        // l % (NS + 1) of {compute, side...}, after the compute stream has
        // cleared the flags word. Several chains are in flight at once, so the latency-bound selection and attention of one
        // layer, and the ramp and tail of each scan, hide under the index
        // scans of the others. No more than kScansInFlight scans run at once
        // (the scan of layer l waits for that of layer l - kScansInFlight):
        // more concurrent scans only make them fight over HBM.
        constexpr int kScansInFlight = 2;
        const int NC = NS + 1;
        if (e == hipSuccess)
            e = hipEventRecord(ev[0], sc);
        for (int k = 0; k < NS && e == hipSuccess; k++)
            e = hipStreamWaitEvent((hipStream_t)side[k], ev[0], 0);
        for (int l = 0; l < n_layers && e == hipSuccess; l++) {
            const int c = l % NC;
            hipStream_t sy = c == 0 ? sc : (hipStream_t)side[c - 1];
            hipEvent_t scanned = ev[1 + NS + l];
            if (l >= kScansInFlight)
                e = hipStreamWaitEvent(sy, ev[1 + NS + l - kScansInFlight], 0);
            if (e == hipSuccess)
                e = score(l, sy);
            if (e == hipSuccess)
                e = hipEventRecord(scanned, sy);
            if (e == hipSuccess)
                e = select(l, sy);
            if (e == hipSuccess)
                e = attend_paged(l, sy);
        }
        // The caller synchronises on the compute stream: join the side streams.
        for (int k = 0; k < NS && e == hipSuccess; k++) {
            e = hipEventRecord(ev[1 + k], (hipStream_t)side[k]);
            if (e == hipSuccess)
                e = hipStreamWaitEvent(sc, ev[1 + k], 0);
        }
        return hip_status(e);
    }

    // Pools in pinned host memory without a hot cache. With no side stream,
    // groups of up to 16 layers one after another (below). With a side
    // stream given: a pipeline over
    // groups of layers of sizes 1, 3, 9, ... (the last takes the rest). The
    // compute stream scores and selects group after group (one launch each
    // per group); the side stream gathers each group's selected rows over
    // PCIe as soon as that group is selected, one launch per group, back to
    // back, so that the PCIe reads hardly stop; once the last gather is done
    // the compute stream attends all layers. Only the first group's scan and
    // selection (one layer) and the attention lie outside the gathers; each
    // group's scan and selection take less time than the gather of the group
    // before it (a layer's scan and selection take about 25 us, its gather
    // about 75 us, so a group may be three times the one before). The gather
    // runs on kPipeGatherWgs workgroups, enough for the PCIe reads, so that
    // the scans beside it keep the other CUs. (Per-layer launches paid a
    // cross-stream wait of 10-20 us per layer, more than they hid; the gather
    // on a full grid starved the scans beside it of CUs.)
    // Hand-overs: the compute stream writes the set's signal after each
    // group's selection and the side stream waits for that value (a wait
    // that is reached first ends about 5 us after the write, an event about
    // 10 us after its record). The side stream records no event between its
    // gathers (a record after a kernel delays the stream's next kernel by
    // 3-5 us), only after the last one, for which the compute stream waits on
    // an event: a signal wait held that long sometimes ended 180 us late.
    const hipStream_t sg = two_streams ? (hipStream_t)side[0] : sc;
    auto staged_tables = [&](int l0, int nl, ScoreLayers &CL, SelectLayers &SL, GatherLayers &GL, AttnLayers &AL) {
        CL.flags = l0 == 0 ? nullptr : flags;      // the first scan clears the word instead
        CL.drop_listed_bs = 1;
        GL.flags = flags;
        AL.flags = flags;
        for (int i = 0; i < nl; i++) {
            const int l = l0 + i;
            const qsa_layer_t &Ly = layers[l];
            CL.keys[i] = Ly.idx_keys;
            CL.scales[i] = Ly.idx_scales;
            CL.q_idx[i] = Ly.q_idx;
            CL.w_idx[i] = Ly.w_idx;
            CL.block_scores[i] = lw[l].bs;
            CL.heads[i] = lw[l].sw.heads;
            CL.lists[i] = lw[l].sw.lists;
            SL.bs[i] = lw[l].bs;
            SL.ws[i] = lw[l].sw;
            SL.sel[i] = lw[l].sel;
            SL.n_sel[i] = lw[l].nsel;
            SL.n_tok[i] = lw[l].ntok;
            GL.sel[i] = lw[l].sel;
            GL.n_sel[i] = lw[l].nsel;
            GL.pt[i] = lw[l].pt;
            GL.pool[i] = pools[l];
            GL.out[i] = lw[l].stage;
            GL.n_tok[i] = lw[l].ntok;
            AL.q[i] = Ly.q;
            AL.rows[i] = static_cast<const uint8_t *>(lw[l].stage);
            AL.n_tok[i] = lw[l].ntok;
            AL.part_o[i] = lw[l].aw.part_o;
            AL.part_lse[i] = lw[l].aw.part_lse;
            AL.out[i] = Ly.out;
        }
    };
    if (!two_streams) {
        // One stream: groups of up to kMaxChainLayers layers, each scanned,
        // selected, gathered (on the whole grid) and attended with one launch
        // per kernel.
        for (int l0 = 0; l0 < n_layers && e == hipSuccess; l0 += kMaxChainLayers) {
            const int nl = n_layers - l0 < kMaxChainLayers ? n_layers - l0 : kMaxChainLayers;
            ScoreLayers CL = {};
            SelectLayers SL = {};
            GatherLayers GL = {};
            AttnLayers AL = {};
            staged_tables(l0, nl, CL, SL, GL, AL);
            e = launch_index_score_layers(CL, nl, batch->ctx_len, batch->idx_row0, batch->n_idx_rows, B,
                                          batch->max_ctx, bs_stride, w.g, K, cfg->sink_blocks, cfg->tail_tokens, sc,
                                          (hipEvent_t)layers[l0].score_events[0],
                                          (hipEvent_t)layers[l0].score_events[1], l0 == 0 ? flags : nullptr);
            if (e == hipSuccess)
                e = launch_select_layers(SL, nl, bs_stride, batch->ctx_len, B, batch->max_ctx, w.g, K,
                                         cfg->sink_blocks, cfg->tail_tokens, sc);
            if (e == hipSuccess)
                e = launch_gather_layers(GL, nl, batch->ctx_len, B, batch->max_ctx, batch->pt_stride,
                                         batch->n_slots, K, cfg->budget_tokens, sc, 0);
            if (e == hipSuccess)
                e = launch_attention_layers(false, AL, nl, 0, 0, B, 0, cfg->budget_tokens, cfg->sm_scale,
                                            lw[l0].aw.tps, sc);
        }
        return hip_status(e);
    }
    int group_len[QSA_MAX_LAYERS];
    int n_groups = 0;
    for (int l0 = 0, want = 1; l0 < n_layers; want *= 3) {
        const int rest = n_layers - l0;
        int nl = want < kMaxChainLayers ? want : kMaxChainLayers;
        nl = nl < rest ? nl : rest;
        if (rest - nl > 0 && rest - nl < nl && rest <= kMaxChainLayers)
            nl = rest;                      // a short remainder joins this group
        group_len[n_groups++] = nl;
        l0 += nl;
    }
    for (int g = 0, l0 = 0; g < n_groups && e == hipSuccess; l0 += group_len[g++]) {
        const int nl = group_len[g];
        ScoreLayers CL = {};
        SelectLayers SL = {};
        GatherLayers GL = {};
        AttnLayers AL = {};
        staged_tables(l0, nl, CL, SL, GL, AL);
        e = launch_index_score_layers(CL, nl, batch->ctx_len, batch->idx_row0, batch->n_idx_rows, B, batch->max_ctx,
                                      bs_stride, w.g, K, cfg->sink_blocks, cfg->tail_tokens, sc,
                                      (hipEvent_t)layers[l0].score_events[0], (hipEvent_t)layers[l0].score_events[1],
                                      l0 == 0 ? flags : nullptr);
        if (e == hipSuccess)
            e = launch_select_layers(SL, nl, bs_stride, batch->ctx_len, B, batch->max_ctx, w.g, K,
                                     cfg->sink_blocks, cfg->tail_tokens, sc);
        // the side stream's wait is enqueued only once the write of its value
        // is, so it can never wait for a value that no write will bring
        if (e == hipSuccess && events->signal) {
            const uint64_t value = events->epoch + 1;
            e = hipStreamWriteValue64(sc, events->signal, value, 0);
            if (e == hipSuccess) {
                events->epoch = value;
                e = hipStreamWaitValue64(sg, events->signal, value, hipStreamWaitValueGte, ~0ull);
            }
        } else if (e == hipSuccess) {
            e = hipEventRecord(ev[1 + NS + l0], sc);
            if (e == hipSuccess)
                e = hipStreamWaitEvent(sg, ev[1 + NS + l0], 0);
        }
        if (e == hipSuccess)
            e = launch_gather_layers(GL, nl, batch->ctx_len, B, batch->max_ctx, batch->pt_stride, batch->n_slots, K,
                                     cfg->budget_tokens, sg, kPipeGatherWgs);
    }
    // The compute stream waits for the last gather (and with it every one
    // before it on the side stream), so the side stream holds no work of this
    // call afterwards; then it attends the layers, up to a group's worth of
    // layers per launch.
    if (e == hipSuccess)
        e = hipEventRecord(ev[0], sg);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(sc, ev[0], 0);
    for (int l0 = 0; l0 < n_layers && e == hipSuccess; l0 += kMaxChainLayers) {
        const int nl = n_layers - l0 < kMaxChainLayers ? n_layers - l0 : kMaxChainLayers;
        ScoreLayers CL = {};
        SelectLayers SL = {};
        GatherLayers GL = {};
        AttnLayers AL = {};
        staged_tables(l0, nl, CL, SL, GL, AL);
        e = launch_attention_layers(false, AL, nl, 0, 0, B, 0, cfg->budget_tokens, cfg->sm_scale, lw[l0].aw.tps, sc);
    }
    return hip_status(e);
}

qsa_status_t qsa_decode_step_static(const qsa_config_t *cfg, const qsa_batch_t *batch, const qsa_layer_t *layers,
                                    int32_t n_layers, qsa_kv_location_t kv_location, qsa_stream_t compute,
                                    const qsa_stream_t *side, int32_t n_side, qsa_step_events_t *events)
{
    qsa_status_t st = check_config(cfg);
    if (st != QSA_OK)
        return st;
    if ((st = check_batch(batch, true, true)) != QSA_OK)
        return st;
    if (n_layers < 1 || n_layers > QSA_MAX_LAYERS ||
        (kv_location != QSA_KV_DEVICE && kv_location != QSA_KV_HOST_PINNED))
        return QSA_ERR_INVALID_ARGUMENT;
    if (make_layout(cfg, batch->batch, batch->max_ctx, n_layers, kv_location).total > QSA_STATIC_SCRATCH_BYTES)
        return QSA_ERR_WORKSPACE_TOO_SMALL;
    void *ws = static_scratch(&st);
    if (!ws)
        return st;
    return qsa_decode_step(cfg, batch, layers, n_layers, kv_location, ws, QSA_STATIC_SCRATCH_BYTES, compute, side,
                           n_side, events);
}

} // extern "C"
