// gather.hip -- page-table translate and row gather.
//
// For every selected token t (ascending), slot = page_table[b][t] and the
// 2048-byte KV row kv_pool[slot] is copied to position p of the staging area
// (article, memory-ledger section: logical token addresses are kept apart
// from physical cache slots; digest, mechanism section: only the selected
// rows are moved, over PCIe when the pool lives in pinned host memory).
// A work unit is the rows of kBlocksPerWg selected C4 blocks; every lane
// moves 16-byte pieces so a row is one contiguous 2 KB burst, which is what
// both HBM and PCIe reads want. One launch may gather several layers (their
// pointers in the kernel arguments), so that the PCIe reads of all of them
// stream without a break, and may run on fewer workgroups than units, each
// taking every G-th unit: the PCIe reads need far fewer waves in flight than
// there are units, and a small gather leaves the other CUs to the kernels
// running beside it.
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int kBlocksPerWg = 4;                       // 16 rows, 32 KB per workgroup
constexpr int kRowsPerWg = kBlocksPerWg * kBT;
constexpr int kPieces = kRowBytes / 16;               // 128 x 16 B per row

// Work unit u = (group x of kBlocksPerWg selection entries, sequence b,
// layer ly), x fastest: workgroup w takes units w, w + G, ... (G workgroups),
// so that a launch may use fewer workgroups than units.
template <int N>
__global__ __launch_bounds__(kThreads) void gather_kernel(const GatherLayersT<N> Ls,
                                                          const int32_t *__restrict__ ctx_len, int max_ctx,
                                                          int64_t pt_stride, int64_t n_slots, int K,
                                                          int budget_tokens, int n_groups, int batch, int n_units)
{
    for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
        const int gx = u % n_groups;
        const int ly = u / (n_groups * batch);
        const int32_t *__restrict__ sel = Ls.sel[ly];
        const int32_t *__restrict__ n_sel = Ls.n_sel[ly];
        const int32_t *__restrict__ pt = Ls.pt[ly];
        const u32x4 *__restrict__ pool = static_cast<const u32x4 *>(Ls.pool[ly]);
        u32x4 *__restrict__ out = static_cast<u32x4 *>(Ls.out[ly]);
        int32_t *__restrict__ n_tok = Ls.n_tok[ly];
        const int b = (u / n_groups) % batch;
        const int L = clamp_ctx(ctx_len[b], max_ctx);
        int ns = n_sel[b];
        ns = ns < 0 ? 0 : (ns > K ? K : ns);
        const int i0 = gx * kBlocksPerWg;
        if (gx == 0 && threadIdx.x == 0 && n_tok) {
            int nt = 0;
            if (ns > 0) {
                const int last = sel[(int64_t)b * K + ns - 1];
                const int end = min(last * kBT + kBT, L);
                nt = (ns - 1) * kBT + (end - last * kBT);
            }
            n_tok[b] = nt;
        }
        if (i0 >= ns)
            continue;                             // uniform

        // 16 rows x 128 pieces = 2048 pieces, 8 per thread; gather all loads first.
        u32x4 v[kRowsPerWg * kPieces / kThreads];
        int64_t dst[kRowsPerWg * kPieces / kThreads];
#pragma unroll
        for (int k = 0; k < kRowsPerWg * kPieces / kThreads; k++) {
            const int c = threadIdx.x + k * kThreads;
            const int r = c / kPieces;            // row within the workgroup
            const int piece = c % kPieces;
            const int i = i0 + r / kBT;           // selection entry
            dst[k] = -1;
            if (i < ns) {
                const int j = sel[(int64_t)b * K + i];
                const int t = j * kBT + (r % kBT);
                if (j >= 0 && t < L) {
                    const int32_t raw = pt[(int64_t)b * pt_stride + t];
                    const int64_t slot = safe_slot(raw, n_slots);
                    if (piece == 0 && slot != raw)
                        raise_flag(Ls.flags, QSA_FLAG_BAD_SLOT);
                    v[k] = __builtin_nontemporal_load(pool + slot * kPieces + piece);
                    const int p = i * kBT + (r % kBT);
                    dst[k] = ((int64_t)b * budget_tokens + p) * kPieces + piece;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kRowsPerWg * kPieces / kThreads; k++)
            if (dst[k] >= 0)
                out[dst[k]] = v[k];
    }
}

} // namespace

template <int N>
static void launch_gather_n(const GatherLayersT<N> &L, int n_layers, const int32_t *ctx_len, int batch, int max_ctx,
                            int64_t pt_stride, int64_t n_slots, int budget_blocks, int budget_tokens, int max_wgs,
                            hipStream_t s)
{
    const int n_groups = (budget_blocks + kBlocksPerWg - 1) / kBlocksPerWg;
    const int n_units = n_groups * batch * n_layers;
    const int grid = max_wgs > 0 && max_wgs < n_units ? max_wgs : n_units;
    hipLaunchKernelGGL((gather_kernel<N>), dim3((unsigned)grid), dim3(kThreads), 0, s, L, ctx_len, max_ctx,
                       pt_stride, n_slots, budget_blocks, budget_tokens, n_groups, batch, n_units);
}

hipError_t launch_gather_layers(const GatherLayers &L, int n_layers, const int32_t *ctx_len, int batch, int max_ctx,
                                int64_t pt_stride, int64_t n_slots, int budget_blocks, int budget_tokens,
                                hipStream_t s, int max_wgs)
{
    if (n_layers < 1 || n_layers > kMaxChainLayers || batch < 1 || budget_blocks < 1)
        return hipErrorInvalidValue;
    if (n_layers > 1) {
        launch_gather_n(L, n_layers, ctx_len, batch, max_ctx, pt_stride, n_slots, budget_blocks, budget_tokens,
                        max_wgs, s);
    } else {
        const GatherLayersT<1> L1 = {{L.sel[0]}, {L.n_sel[0]}, {L.pt[0]}, {L.pool[0]},
                                     {L.out[0]}, {L.n_tok[0]}, L.flags};
        launch_gather_n(L1, 1, ctx_len, batch, max_ctx, pt_stride, n_slots, budget_blocks, budget_tokens, max_wgs,
                        s);
    }
    return hipGetLastError();
}

hipError_t launch_gather(const int32_t *sel, const int32_t *n_sel, const int32_t *ctx_len, int batch, int max_ctx,
                         const int32_t *pt, int64_t pt_stride, int64_t n_slots, const void *pool, void *out,
                         int budget_blocks, int budget_tokens, int32_t *n_tok, uint32_t *flags, hipStream_t s)
{
    GatherLayers L = {};
    L.flags = flags;
    L.sel[0] = sel;
    L.n_sel[0] = n_sel;
    L.pt[0] = pt;
    L.pool[0] = pool;
    L.out[0] = out;
    L.n_tok[0] = n_tok;
    return launch_gather_layers(L, 1, ctx_len, batch, max_ctx, pt_stride, n_slots, budget_blocks, budget_tokens, s);
}

} // namespace qsa
