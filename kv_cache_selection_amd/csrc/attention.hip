// attention.hip -- split-K GQA decode attention over the selected rows and the
// log-sum-exp merge of the splits.
//
// For query head h with KV head g = h / 8 and the selected tokens T:
//     z_t = sm_scale * (q_h . K_{g,t}),   out_h = sum_t softmax(z)_t V_{g,t}
// (the attention the article's "fast path" computes, restricted to the
// gathered set). The tokens are split into chunks of 64 or 128 (kTPSMin or
// kTPS, whichever gives the launch enough workgroups); a workgroup (split s,
// sequence b, layer of the launch) attends all 16 query heads over its chunk,
// each wave over 16 or 32 tokens, and writes the normalised partial outputs
// and their log-sum-exp; the merge kernel combines the splits exactly:
// out = sum_s e^{lse_s - LSE} O_s. One workgroup reads each token's whole
// 2 KB row (K and V of both KV heads).
//
// Per wave, for each chunk of 16 tokens:
//  - all K and V rows of the chunk are requested before the first multiply;
//  - QK^T on the matrix cores: v_mfma_f32_16x16x32_bf16 with A = the 16 query
//    heads (rows 0..7 the heads of KV head 0, rows 8..15 those of KV head 1)
//    and B = 32 dims x 16 tokens of K_g read straight from the rows (each
//    lane loads 16 contiguous bytes of one token's K), one chain per KV head;
//    of each chain's output the rows of its own heads are kept;
//  - the softmax in fp32, the statistics reduced across the 16 lanes that
//    hold one head's scores with DPP row operations, and rescaled online
//    between the chunks;
//  - PV on the matrix cores as well (v_mfma_f32_16x16x32_bf16, the two KV
//    heads stacked along k: 16 tokens under V_0, then the same 16 under V_1):
//    the V rows go through LDS, where ds_read_b64_tr_b16 reads them
//    transposed (k = tokens), and P enters as an exact bf16 high part plus a
//    bf16 remainder (16 mantissa bits), zero outside its own KV head's k
//    range, so both heads accumulate into the same 16-row output tiles.
// The four waves of a workgroup then merge their partial states in LDS.
//
// Rows come either from the staging area (qsa_sparse_decode, the pinned-host
// path) or straight from the KV pool through the page table (the gather is
// fused into the attention when the pool is in HBM). One launch may cover
// several layers: their pointers travel in the kernel arguments.
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 16;                          // tokens per MFMA tile (one chunk of a wave)
static_assert(kWaves * kTile * 2 == kTPS && kWaves * kTile == kTPSMin, "tokens per split: 1 or 2 chunks a wave");
constexpr int kKBytes = kDh * 2;                   // 512 bytes of K (or V) per head per row
constexpr int kVBytes = kHkv * kKBytes;            // a token's V: both heads, 1 KB
// A wave's V tile in LDS: 16 token rows of 1 KB (V of head 0, then head 1),
// 32 bytes of padding between rows so that the transposing reads of 4 rows
// hit distinct banks.
constexpr int kVPitch = kVBytes + 32;
constexpr int kVTileBytes = kTile * kVPitch;       // 16,896
constexpr int kOBytes = kWaves * kHq * kDh * 4;    // per-wave partial outputs for the merge (64 KB)
constexpr int kSmemBytes = kWaves * kVTileBytes > kOBytes ? kWaves * kVTileBytes : kOBytes;

// Max / sum over the 16 lanes of a DPP row (lanes 16r .. 16r + 15): swaps
// within pairs and quads, then the half-row and row mirrors.
template <bool kMax>
__device__ __forceinline__ float row16_reduce(float x)
{
    auto op = [](float a, float b) { return kMax ? fmaxf(a, b) : a + b; };
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));  // quad_perm 1,0,3,2
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));  // quad_perm 2,3,0,1
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false))); // row_half_mirror
    x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false))); // row_mirror
    return x;
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The exact split of p into a bf16 high part and a bf16 remainder, as the
// halves of two packed pairs (elements e, e+1 of each).
__device__ __forceinline__ void split_pair(float p0, float p1, uint32_t &hi, uint32_t &lo)
{
    const uint32_t h0 = __float_as_uint(p0) & 0xFFFF0000u;
    const uint32_t h1 = __float_as_uint(p1) & 0xFFFF0000u;
    const uint32_t l0 = __float_as_uint(p0 - __uint_as_float(h0)) >> 16;
    const uint32_t l1 = __float_as_uint(p1 - __uint_as_float(h1)) & 0xFFFF0000u;
    hi = (h0 >> 16) | h1;
    lo = l0 | l1;
}

// Grid (n_split, layers, B): workgroup (split s, layer ly, sequence b)
// attends all 16 query heads over the split's 64 kChunks tokens, so that each
// token's whole 2 KB row is read by one wave (whole rows stream about 13 %
// faster than the four 512-byte pieces of two workgroups). Each wave takes
// kChunks chunks of 16 tokens, one after the other.
// Two waves per SIMD (two workgroups per CU): a register budget of 256.
template <bool kPaged, int N, int kChunks>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_split_kernel(const AttnLayersT<N> Ls, int64_t pt_stride, int max_ctx, int budget_blocks, int budget_tokens,
                       float sm_scale, int n_split)
{
    const int ly = blockIdx.y;
    const uint16_t *__restrict__ q = Ls.q[ly];
    const uint8_t *__restrict__ rows = Ls.rows[ly];
    const int32_t *__restrict__ pt = Ls.pt[ly];
    const int64_t n_slots = Ls.n_slots[ly];
    const int32_t *__restrict__ sel = Ls.sel[ly];
    const int32_t *__restrict__ n_tok = Ls.n_tok[ly];
    float *__restrict__ part_o = Ls.part_o[ly];
    float *__restrict__ part_lse = Ls.part_lse[ly];
    __shared__ __attribute__((aligned(16))) float ps[kWaves][kHq][kTile];  // the chunk's probabilities
    __shared__ float sstat[kWaves][kHq][2];         // per-wave (max, sum) for the workgroup merge
    __shared__ float swt[kWaves][kHq];              // per-wave weights exp(m_w - M) of each head
    __shared__ float sden[kHq];                     // each head's normaliser
    // V tiles during the token loop, then the per-wave partial outputs
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];

    const int s = blockIdx.x;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4;
    const int col = lane & 15;

    constexpr int kWaveTok = kTile * kChunks;
    const int split_p0 = s * kWaves * kWaveTok;
    const int wave_p0 = split_p0 + wave * kWaveTok;

    // Everything that does not depend on the token count is requested at
    // once: the count, the query, and each lane's row for its K token (lane
    // l holds token l & 15 of each chunk). On the paged path the row is the
    // page-table slot of the selected token; indices are clamped so that
    // every read stays inside its buffer before the count is known.
    // The loads are unconditional (selects come after them), so that the
    // compiler can count them: the selection entries of both chunks and the
    // query go out together, then the page-table slots of both chunks.
    int nt = n_tok[b];
    int64_t row_k[kChunks];
    int ptok[kChunks], stok[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; c++) {
        const int p = min(wave_p0 + kTile * c + col, budget_tokens - 1);
        ptok[c] = p;
        if (kPaged)
            stok[c] = sel[(int64_t)b * budget_blocks + (p >> 2)];
    }
    // A operand of QK^T: lane holds query head (lane & 15), dims
    // 32 kk + 8 (lane >> 4) .. +8 for MFMA kk. Rows 0..7 are the heads of KV
    // head 0, rows 8..15 those of KV head 1.
    bf16x8 qa[kDh / 32];
    {
        const uint16_t *qr = q + ((int64_t)b * kHq + col) * kDh + 8 * grp;
#pragma unroll
        for (int kk = 0; kk < kDh / 32; kk++)
            qa[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qr + 32 * kk));
    }
    if (kPaged) {
        // token t of the selection; a block index outside the context (only
        // in entries past the count) reads slot 0. With no context the table
        // may be empty, so a selection entry is read instead.
        int32_t slot[kChunks];
        bool in[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; c++) {
            const int t = stok[c] * kBT + (ptok[c] & 3);
            in[c] = t >= 0 && max_ctx > 0;
            const int tc = min(max(t, 0), max_ctx - 1);
            const int32_t *src = max_ctx > 0 ? pt + (int64_t)b * pt_stride + tc : sel + (int64_t)b * budget_blocks;
            slot[c] = *src;
        }
        // every slot is used here, so all the reads are issued before any
        // is waited for (not moved into the branches of the selects below)
#pragma unroll
        for (int c = 0; c < kChunks; c++)
            asm volatile("" : "+v"(slot[c]));
#pragma unroll
        for (int c = 0; c < kChunks; c++) {
            row_k[c] = in[c] ? safe_slot(slot[c], n_slots) : 0;
            // a selected token (p < n_tok) whose entry is outside the pool
            if (in[c] && row_k[c] != slot[c] && ptok[c] < nt && grp == 0)
                raise_flag(Ls.flags, QSA_FLAG_BAD_SLOT);
        }
    } else {
#pragma unroll
        for (int c = 0; c < kChunks; c++)
            row_k[c] = (int64_t)b * budget_tokens + ptok[c];
    }

    if (!kPaged && s == 0 && tid == 0 && (nt < 0 || nt > budget_tokens))
        raise_flag(Ls.flags, QSA_FLAG_BAD_N_TOK);
    nt = nt < 0 ? 0 : (nt > budget_tokens ? budget_tokens : nt);
    const int64_t part_base = (int64_t)b * kHq * n_split + s;   // head 0, split s
    if (split_p0 >= nt) {
        if (tid < kHq)
            part_lse[part_base + (int64_t)tid * n_split] = -INFINITY;
        return;
    }

    // Softmax state of the wave: lane l holds heads 4 (l >> 4) + v, the rows
    // of the C tiles it holds, for QK^T and PV alike; the state runs over
    // the wave's two chunks (online rescale).
    float m_run[4], l_run[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        m_run[v] = -INFINITY;
        l_run[v] = 0.0f;
    }
    // Output accumulators, the C tiles of PV: o[m][v] = head 4 (l >> 4) + v,
    // dim 16 m + (l & 15).
    f32x4 o[kDh / 16];
#pragma unroll
    for (int m = 0; m < kDh / 16; m++)
        o[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    uint8_t *vt = smem + wave * kVTileBytes;

    if (wave_p0 < nt) {                             // uniform: the wave has valid tokens
#pragma unroll
        for (int c = 0; c < kChunks; c++) {
            const int c_p0 = wave_p0 + kTile * c;
            // The chunk's rows: K of both heads (lane: 16 B of each of 16
            // pieces of its token's K), then V of both heads (one token's
            // 1 KB per load, lane: 16 B). Every request is made, also for
            // tokens past the count (rows clamped to valid ones, masked
            // below), so the compiler can count them; QK^T waits for the K
            // rows only.
            u32x4 kd[kHkv][kDh / 32];
            u32x4 vd[kTile];
            const uint8_t *rk = rows + row_k[c] * kRowBytes + 16 * grp;
#pragma unroll
            for (int g = 0; g < kHkv; g++)
#pragma unroll
                for (int kk = 0; kk < kDh / 32; kk++)
                    kd[g][kk] = *reinterpret_cast<const u32x4 *>(rk + g * kKBytes + 64 * kk);
            const uint32_t rlo = (uint32_t)row_k[c], rhi = (uint32_t)(row_k[c] >> 32);
#pragma unroll
            for (int t = 0; t < kTile; t++) {
                // uniform across the wave: token c_p0 + t, whose row lane t holds
                const int64_t r = (int64_t)(((uint64_t)__builtin_amdgcn_readlane(rhi, t) << 32) |
                                            __builtin_amdgcn_readlane(rlo, t));
                vd[t] = *reinterpret_cast<const u32x4 *>(rows + r * kRowBytes + kHkv * kKBytes + 16 * lane);
            }
            // QK^T: acc[g] rows 8 g .. 8 g + 7 are the heads of KV head g.
            f32x4 acc[kHkv];
#pragma unroll
            for (int g = 0; g < kHkv; g++) {
                acc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < kDh / 32; kk++)
                    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], __builtin_bit_cast(bf16x8, kd[g][kk]),
                                                                     acc[g], 0, 0, 0);
            }
            // Lane l: heads 4 (l >> 4) + v (group l >> 5), token c_p0 + (l & 15).
            const bool valid = c_p0 + col < nt;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float z = valid ? (lane < 32 ? acc[0][v] : acc[1][v]) * sm_scale : -INFINITY;
                const float mx = fmaxf(m_run[v], row16_reduce<true>(z));   // finite: token c_p0 is valid
                const float r = __expf(m_run[v] - mx);                     // 0 on the first chunk
                float e = valid ? __expf(z - mx) : 0.0f;
                // Keep 16 mantissa bits (a bf16 head plus a bf16 remainder),
                // the precision PV uses, so that numerator and normaliser agree.
                const uint32_t hb = __float_as_uint(e) & 0xFFFF0000u;
                const uint32_t lb = __float_as_uint(e - __uint_as_float(hb)) & 0xFFFF0000u;
                e = __uint_as_float(hb) + __uint_as_float(lb);
                l_run[v] = l_run[v] * r + row16_reduce<false>(e);
                m_run[v] = mx;
#pragma unroll
                for (int m = 0; m < kDh / 16; m++)
                    o[m][v] *= r;
                ps[wave][4 * grp + v][col] = e;
            }
            // V rows to LDS (row t), zero past the count
#pragma unroll
            for (int t = 0; t < kTile; t++)
                *reinterpret_cast<u32x4 *>(vt + t * kVPitch + 16 * lane) =
                    c_p0 + t < nt ? vd[t] : u32x4{0u, 0u, 0u, 0u};
            wave_lds_sync();

            // PV on the matrix cores, v_mfma_f32_16x16x32_bf16 per 16 dims,
            // with both KV heads stacked along k: k = 0..15 are the chunk's
            // tokens under V_0, k = 16..31 the same tokens under V_1.
            //  A = P: lane l holds row (head) `col`, k = 8 (l >> 4) .. +7, i.e.
            //      tokens 8 ((l >> 4) & 1) .. +7 of KV head g = l >> 5; zero
            //      unless head `col` belongs to g (then the product picks
            //      V_g for the heads of g only). P enters as its exact split
            //      into a bf16 high part and a bf16 remainder.
            //  B = V: lane l holds k = 8 (l >> 4) .. +7 and column (dim)
            //      16 m + col, read transposed from the rows in LDS, four
            //      tokens per read: in each group of 16 lanes, lane j supplies
            //      the address of token row base + (j >> 2), dims 4 (j & 3)
            //      .. +3 of V_g, and lane c receives dim c of the four rows.
            const int g_k = lane >> 5;                  // the KV head of this lane's k range
            const int tok0 = 8 * (grp & 1);             // its first token
            bf16x8 a_hi, a_lo;
            {
                uint32_t hi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
                if ((col >> 3) == g_k) {
                    const f32x4 p0 = *reinterpret_cast<const f32x4 *>(&ps[wave][col][tok0]);
                    const f32x4 p1 = *reinterpret_cast<const f32x4 *>(&ps[wave][col][tok0 + 4]);
                    split_pair(p0[0], p0[1], hi[0], lo[0]);
                    split_pair(p0[2], p0[3], hi[1], lo[1]);
                    split_pair(p1[0], p1[1], hi[2], lo[2]);
                    split_pair(p1[2], p1[3], hi[3], lo[3]);
                }
                a_hi = __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
                a_lo = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
            }
            const uint8_t *vrd = vt + (tok0 + (col >> 2)) * kVPitch + g_k * kKBytes + 8 * (col & 3);
#pragma unroll
            for (int m = 0; m < kDh / 16; m++) {
                const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(vrd + 32 * m));
                const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(vrd + 4 * kVPitch + 32 * m));
                const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
                o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, bv, o[m], 0, 0, 0);
                o[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, bv, o[m], 0, 0, 0);
            }
            // the next chunk's V overwrites this chunk's tile
            wave_lds_sync();
        }
    }

    // Workgroup merge of the four waves' states (the V tiles' LDS is reused):
    // each wave's accumulators go to LDS as [dim][head], 16 bytes (4 heads of
    // one dim) per store; 16 threads then work out each head's wave weights
    // f_w = exp(m_w - M), normaliser and LSE once, and every thread combines
    // one dim for the 16 heads.
    __syncthreads();
    float(*sod)[kDh][kHq] = reinterpret_cast<float(*)[kDh][kHq]>(smem);
#pragma unroll
    for (int m = 0; m < kDh / 16; m++)
        *reinterpret_cast<f32x4 *>(&sod[wave][16 * m + col][4 * grp]) = o[m];
    if (col == 0) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            sstat[wave][4 * grp + v][0] = m_run[v];
            sstat[wave][4 * grp + v][1] = l_run[v];
        }
    }
    __syncthreads();
    if (tid < kHq) {
        const int h = tid;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++)
            M = fmaxf(M, sstat[w][h][0]);
        float den = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float mw = sstat[w][h][0];
            const float f = (mw == -INFINITY) ? 0.0f : __expf(mw - M);
            swt[w][h] = f;
            den += f * sstat[w][h][1];
        }
        sden[h] = den;
        part_lse[part_base + (int64_t)h * n_split] = M + logf(den);
    }
    __syncthreads();
    for (int d = tid; d < kDh; d += kThreads) {
        float acc[kHq];
#pragma unroll
        for (int h = 0; h < kHq; h++)
            acc[h] = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
#pragma unroll
            for (int h4 = 0; h4 < kHq; h4 += 4) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&sod[w][d][h4]);
#pragma unroll
                for (int h = 0; h < 4; h++)
                    acc[h4 + h] = fmaf(swt[w][h4 + h], a[h], acc[h4 + h]);
            }
        }
#pragma unroll
        for (int h = 0; h < kHq; h++)
            part_o[(part_base + (int64_t)h * n_split) * kDh + d] = acc[h] / sden[h];
    }
}

// One workgroup per (sequence, head) and layer (grid (B * kHq, layers));
// thread d owns output dim d. Every thread reads the (uniform) split LSEs
// itself and its column of partial outputs in batches of kBatch splits (16
// when the launch has at most 16 splits, else 32), so that up to 32 splits
// take one round of loads: for each batch, the running max is raised and
// the sums rescaled.
template <int N, int kBatch>
__global__ __launch_bounds__(kDh) void merge_kernel(const AttnLayersT<N> Ls, int n_split)
{
    const float *__restrict__ part_o = Ls.part_o[blockIdx.y];
    const float *__restrict__ part_lse = Ls.part_lse[blockIdx.y];
    float *__restrict__ out = Ls.out[blockIdx.y];
    const int bh = blockIdx.x;              // b * kHq + h
    const int tid = threadIdx.x;
    const float *lse = part_lse + (int64_t)bh * n_split;
    const float *col = part_o + (int64_t)bh * n_split * kDh + tid;
    float M = -INFINITY, acc = 0.0f, den = 0.0f;
    for (int s0 = 0; s0 < n_split; s0 += kBatch) {
        float ls[kBatch], x[kBatch];
        // unconditional loads of clamped splits (no branches between them,
        // so all are in flight together), masked afterwards
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            const int sc = min(s0 + u, n_split - 1);
            ls[u] = lse[sc];
            x[u] = col[(int64_t)sc * kDh];
        }
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            const bool in = s0 + u < n_split;
            ls[u] = in ? ls[u] : -INFINITY;
            x[u] = in ? x[u] : 0.0f;
        }
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < kBatch; u++)
            mb = fmaxf(mb, ls[u]);
        if (mb == -INFINITY)
            continue;                       // uniform: every split of the batch is empty
        const float Mn = fmaxf(M, mb);
        const float r = __expf(M - Mn);     // 0 while M is still -inf
        acc *= r;
        den *= r;
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            const float ws = ls[u] == -INFINITY ? 0.0f : __expf(ls[u] - Mn);
            den += ws;
            // empty splits hold stale data: select, not multiply
            acc = ws != 0.0f ? fmaf(ws, x[u], acc) : acc;
        }
        M = Mn;
    }
    out[(int64_t)bh * kDh + tid] = den > 0.0f ? acc / den : 0.0f;
}

} // namespace

template <int N>
static hipError_t launch_attention_n(bool paged, const AttnLayersT<N> &L, int n_layers, int64_t pt_stride,
                                     int max_ctx, int batch, int budget_blocks, int budget_tokens, float sm_scale,
                                     int tps, hipStream_t s)
{
    if (tps != kTPS && tps != kTPSMin)
        return hipErrorInvalidValue;
    const bool big = tps == kTPS;
    const int n_split = (budget_tokens + tps - 1) / tps;
    dim3 grid((unsigned)n_split, (unsigned)n_layers, (unsigned)batch);
    if (paged && big)
        hipLaunchKernelGGL((attn_split_kernel<true, N, 2>), grid, dim3(kThreads), 0, s, L, pt_stride, max_ctx,
                           budget_blocks, budget_tokens, sm_scale, n_split);
    else if (paged)
        hipLaunchKernelGGL((attn_split_kernel<true, N, 1>), grid, dim3(kThreads), 0, s, L, pt_stride, max_ctx,
                           budget_blocks, budget_tokens, sm_scale, n_split);
    else if (big)
        hipLaunchKernelGGL((attn_split_kernel<false, N, 2>), grid, dim3(kThreads), 0, s, L, pt_stride, max_ctx,
                           budget_blocks, budget_tokens, sm_scale, n_split);
    else
        hipLaunchKernelGGL((attn_split_kernel<false, N, 1>), grid, dim3(kThreads), 0, s, L, pt_stride, max_ctx,
                           budget_blocks, budget_tokens, sm_scale, n_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const dim3 mgrid((unsigned)(batch * kHq), (unsigned)n_layers);
    if (n_split <= 16)
        hipLaunchKernelGGL((merge_kernel<N, 16>), mgrid, dim3(kDh), 0, s, L, n_split);
    else
        hipLaunchKernelGGL((merge_kernel<N, 32>), mgrid, dim3(kDh), 0, s, L, n_split);
    return hipGetLastError();
}

hipError_t launch_attention_layers(bool paged, const AttnLayers &L, int n_layers, int64_t pt_stride, int max_ctx,
                                   int batch, int budget_blocks, int budget_tokens, float sm_scale, int tps,
                                   hipStream_t s)
{
    if (n_layers < 1 || n_layers > kMaxChainLayers)
        return hipErrorInvalidValue;
    if (n_layers > 1)
        return launch_attention_n(paged, L, n_layers, pt_stride, max_ctx, batch, budget_blocks, budget_tokens,
                                  sm_scale, tps, s);
    const AttnLayersT<1> L1 = {{L.q[0]},     {L.rows[0]},   {L.pt[0]},       {L.n_slots[0]}, {L.sel[0]},
                               {L.n_tok[0]}, {L.part_o[0]}, {L.part_lse[0]}, {L.out[0]},     L.flags};
    return launch_attention_n(paged, L1, 1, pt_stride, max_ctx, batch, budget_blocks, budget_tokens, sm_scale,
                              tps, s);
}

hipError_t launch_attention_staged(const uint16_t *q, const void *kv, const int32_t *n_tok, int batch,
                                   int budget_tokens, float sm_scale, const AttnWs &ws, float *out, hipStream_t s)
{
    AttnLayers L = {};
    L.flags = ws.flags;
    L.q[0] = q;
    L.rows[0] = static_cast<const uint8_t *>(kv);
    L.n_tok[0] = n_tok;
    L.part_o[0] = ws.part_o;
    L.part_lse[0] = ws.part_lse;
    L.out[0] = out;
    return launch_attention_layers(false, L, 1, 0, 0, batch, 0, budget_tokens, sm_scale, ws.tps, s);
}

hipError_t launch_attention_paged(const uint16_t *q, const void *pool, const int32_t *pt, int64_t pt_stride,
                                  int64_t n_slots, const int32_t *sel, const int32_t *n_tok, const int32_t *ctx_len,
                                  int max_ctx, int batch, int budget_blocks, int budget_tokens, float sm_scale,
                                  const AttnWs &ws, float *out, hipStream_t s)
{
    (void)ctx_len;
    AttnLayers L = {};
    L.flags = ws.flags;
    L.q[0] = q;
    L.rows[0] = static_cast<const uint8_t *>(pool);
    L.pt[0] = pt;
    L.n_slots[0] = n_slots;
    L.sel[0] = sel;
    L.n_tok[0] = n_tok;
    L.part_o[0] = ws.part_o;
    L.part_lse[0] = ws.part_lse;
    L.out[0] = out;
    return launch_attention_layers(true, L, 1, pt_stride, max_ctx, batch, budget_blocks, budget_tokens, sm_scale,
                                   ws.tps, s);
}

} // namespace qsa
