// multiscore.hip -- indexer scoring of several queries per sequence at once
// (prefill or chunked decode).
//
// Each of Q queries of sequence b scores the index with the single-query
// formula (digest page, mechanism section; the workload's score):
//     s_{i,t} = sum_h w_{i,h} * ReLU(sigma_t * (q_{i,h} . k_t)),
// causally: query i sees the tokens t <= pos[i]. Its C4 block scores are the
// max over the block's visible tokens, -inf for a block it does not see.
//
// With many queries the scan becomes a dense contraction,
// [4Q x 64] (queries x heads, by dims) times [64 x L] (dims by tokens), so it
// runs on the matrix cores with real operands: for a group of 16 tokens the
// widened keys are the B operand of v_mfma_f32_16x16x32_bf16 exactly as in
// the single-query kernel (lane l holds 16 bytes of token l & 15), and each
// row block of A holds 4 queries x 4 heads, so one pair of MFMAs gives lane l
// the four heads of query 4 r + (l >> 4) for token l & 15. Per token the
// kernel reads 66 bytes and writes Q bytes of block scores (one fp32 per four
// tokens per query), and does 512 Q flops.
#include "qsa_internal.h"

#include <type_traits>

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int kTile = 256;                 // tokens per workgroup iteration
constexpr int kGroups = kTile / 16;        // 16-token MFMA column groups per tile

// Widened keys of one tile in LDS: plane h (dims 16 j + 8 h + 0..7), slice j,
// token t at kw[h][j][t ^ 2 j]. The xor makes the loader's writes (four
// slices of two tokens per eight lanes) and the readers' 16-byte reads
// (eight consecutive tokens of one slice) hit distinct banks.
__device__ __forceinline__ int kw_index(int j, int t)
{
    return j * kTile + (t ^ (2 * j));
}

// max(a, b) for values that are never NaN, as med3(a, b, pinf) with pinf an
// opaque +inf: unlike fmaxf it needs no canonicalisation of a DPP-moved
// operand, and the compiler cannot turn it back into fmaxf.
__device__ __forceinline__ float max_nn(float a, float b, float pinf)
{
    return __builtin_amdgcn_fmed3f(a, b, pinf);
}

// the value of lane l ^ 1 (ctrl 0xB1) or l ^ 2 (ctrl 0x4E)
template <int CTRL>
__device__ __forceinline__ float quad_swap(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Grid (chunks of chunk_tokens, a multiple of kTile; B). Each iteration the
// workgroup's 256 threads load the next tile's 16 KB of codes (1 KB per
// instruction, lane l: token 16 i + l / 4 of the wave's 64, bytes 16 (l & 3)),
// widen them once into LDS, and the four waves split the tile's contraction:
// WQ waves over the RB row blocks of 4 queries, 4 / WQ over its tokens.
//
// sigma_t enters as |sigma_t| times the dot products with the key's signs
// flipped when sigma_t < 0 (the flip is exact), so the score of a query-token
// pair is |sigma_t| * sum_h w_h max(q_h . k'_t, 0): nine VALU operations
// per pair of MFMAs. The C4 block max over a lane quad is taken for four
// column groups at once as a reduce-scatter (two exchanges over lane ^ 2,
// one over lane ^ 1), after which lane p of the quad holds group p's block,
// so block scores reach LDS as one full-wave write per four groups and
// leave it as rows of 64 floats per query and tile. Tiles that every query
// sees in full skip the causal and length mask.
template <int RB>
__global__ __launch_bounds__(kThreads) void multi_score_kernel(
    const uint8_t *__restrict__ keys, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ q_idx,
    const float *__restrict__ w_idx, const int32_t *__restrict__ q_pos, const int32_t *__restrict__ ctx_len,
    const int64_t *__restrict__ row0, int64_t n_rows, int max_ctx, int chunk_tokens, float *__restrict__ out,
    int64_t bs_stride)
{
    constexpr int Q = 4 * RB;
    constexpr int WQ = RB >= 4 ? 4 : RB;   // waves across row blocks
    constexpr int WT = 4 / WQ;             // waves across the tile's tokens
    constexpr int RBW = RB / WQ;           // row blocks per wave
    constexpr int GPW = kGroups / WT;      // column groups per wave
    // Block scores of the tile, row qi at column c ^ (16 (qi & 1)): a wave's
    // write covers 16 columns of four rows, and the xor puts rows 2m and
    // 2m + 1 on different halves of the banks.
    constexpr int kStage = kTile / kBT;
    __shared__ u32x4 kw[2][4 * kTile];
    __shared__ float sig[kTile];
    __shared__ float stage[Q][kStage];
    __shared__ int32_t posq[Q];
    __shared__ int32_t pos_min;

    const int b = blockIdx.y;
    const int64_t r0 = row0[b];
    int L = clamp_ctx(ctx_len[b], max_ctx);
    if (r0 < 0 || r0 + L > n_rows)
        L = 0;
    const int t_begin = blockIdx.x * chunk_tokens;
    if (t_begin >= L)
        return;
    const int n_blk = (L + kBT - 1) / kBT;
    const int t_end = min(t_begin + chunk_tokens, L);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint8_t *kbase = keys + r0 * kIdxD;
    const uint16_t *sbase = scales + r0;

    // loader mapping
    const int ld_j = lane & 3;
    const int ld_t = 64 * wave + (lane >> 2);
    u32x4 kn[4];
    uint16_t sn[4];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = t0 + ld_t + 16 * i;
            kn[i] = t < L ? __builtin_nontemporal_load(
                                reinterpret_cast<const u32x4 *>(kbase + (int64_t)t * kIdxD + 16 * ld_j))
                          : u32x4{0u, 0u, 0u, 0u};
            sn[i] = t < L ? sbase[t] : (uint16_t)0;
        }
    };
    load_tile(t_begin);

    if (tid < Q)
        posq[tid] = q_pos[(int64_t)b * Q + tid];
    __syncthreads();
    if (tid < 64) {
        int m = tid < Q ? posq[tid] : INT32_MAX;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            m = min(m, __shfl_xor(m, o));
        if (tid == 0)
            pos_min = m;
    }

    // This wave's row blocks and column groups.
    const int rb0 = (wave % WQ) * RBW;
    const int g0 = (wave / WQ) * GPW;
    // A operands: row block r, lane l: row l & 15 = query 4 r + ((l & 15) >> 2),
    // head l & 3; dims 16 (l >> 4) + 0..7 for the first MFMA, + 8..15 for the
    // second, matching the B operand's lane layout. The lane's outputs belong
    // to query 4 r + (l >> 4), whose weights and position it keeps.
    bf16x8 qa[RBW][2];
    f32x4 wv[RBW];
    int pq[RBW];
#pragma unroll
    for (int r = 0; r < RBW; r++) {
        const int qa_i = 4 * (rb0 + r) + ((lane & 15) >> 2);
        const u32x4 *qrow = reinterpret_cast<const u32x4 *>(
            q_idx + (((int64_t)b * Q + qa_i) * kIdxH + (lane & 3)) * kIdxD + 16 * (lane >> 4));
        qa[r][0] = __builtin_bit_cast(bf16x8, qrow[0]);
        qa[r][1] = __builtin_bit_cast(bf16x8, qrow[1]);
        const int qi = 4 * (rb0 + r) + (lane >> 4);
        wv[r] = *reinterpret_cast<const f32x4 *>(w_idx + ((int64_t)b * Q + qi) * kIdxH);
        pq[r] = posq[qi];
    }
    // Use the operands once here, so the wait for their loads is placed
    // before the loop. Otherwise the compiler waits for them inside the
    // scoring pass of every tile, where the same counter also covers the next
    // tile's prefetch, and that prefetch stops overlapping the pass.
#pragma unroll
    for (int r = 0; r < RBW; r++)
        asm volatile("" ::"v"(qa[r][0]), "v"(qa[r][1]), "v"(wv[r]));

    float pinf;
    asm volatile("v_mov_b32 %0, 0x7f800000" : "=v"(pinf));
    const bool hi2 = lane & 2, hi1 = lane & 1;

    auto score_tile = [&](int t0, auto masked) {
        float sv[RBW][4];
#pragma unroll
        for (int g = 0; g < GPW; g++) {
            const int tl = 16 * (g0 + g) + (lane & 15);     // token in the tile
            const int x = kw_index(lane >> 4, tl);
            const bf16x8 kb0 = __builtin_bit_cast(bf16x8, kw[0][x]);
            const bf16x8 kb1 = __builtin_bit_cast(bf16x8, kw[1][x]);
            const float sigma = sig[tl];
            f32x4 acc[RBW];
#pragma unroll
            for (int r = 0; r < RBW; r++) {
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[r][0], kb0, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[r][1], kb1, acc[r], 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < RBW; r++) {
                // acc[r][h] = q_{i,h} . k'_t, i = 4 (rb0 + r) + (l >> 4), t = t0 + tl
                // ReLU as med3(x, 0, +inf): fmaxf would first canonicalise the MFMA result
                float s = wv[r][0] * max_nn(acc[r][0], 0.0f, pinf);
                s = fmaf(wv[r][1], max_nn(acc[r][1], 0.0f, pinf), s);
                s = fmaf(wv[r][2], max_nn(acc[r][2], 0.0f, pinf), s);
                s = fmaf(wv[r][3], max_nn(acc[r][3], 0.0f, pinf), s);
                s *= sigma;
                if (decltype(masked)::value) {
                    const int t = t0 + tl;
                    s = (t < L && t <= pq[r]) ? s : -INFINITY;
                }
                sv[r][g & 3] = s;
            }
            if ((g & 3) == 3) {
#pragma unroll
                for (int r = 0; r < RBW; r++) {
                    // lane p keeps groups (p & 2) + {0, 1}, maxed with lane p ^ 2
                    float ka = hi2 ? sv[r][2] : sv[r][0];
                    float kb = hi2 ? sv[r][3] : sv[r][1];
                    const float sa = hi2 ? sv[r][0] : sv[r][2];
                    const float sb = hi2 ? sv[r][1] : sv[r][3];
                    ka = max_nn(ka, quad_swap<0x4E>(sa), pinf);
                    kb = max_nn(kb, quad_swap<0x4E>(sb), pinf);
                    // then group p, maxed with lane p ^ 1
                    const float k = max_nn(hi1 ? kb : ka, quad_swap<0xB1>(hi1 ? ka : kb), pinf);
                    const int qi = 4 * (rb0 + r) + (lane >> 4);
                    stage[qi][(4 * (g0 + g - 3 + (lane & 3)) + ((lane & 15) >> 2)) ^ (16 * (qi & 1))] = k;
                }
            }
        }
    };

    float *out_b = out + (int64_t)b * Q * bs_stride;
    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
        // this tile's codes, widened, signs flipped with sigma's, into LDS
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int x = kw_index(ld_j, ld_t + 16 * i);
            const uint32_t flip = (sn[i] & 0x8000u) ? 0x80008000u : 0u;
            u32x4 lo = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(kn[i].x, kn[i].y));
            u32x4 hi = __builtin_bit_cast(u32x4, e4m3x8_to_bf16x8(kn[i].z, kn[i].w));
            kw[0][x] = lo ^ flip;
            kw[1][x] = hi ^ flip;
            if (ld_j == 0)
                sig[ld_t + 16 * i] = fabsf((float)__builtin_bit_cast(_Float16, sn[i]));
        }
        __syncthreads();
        if (t0 + kTile < t_end)
            load_tile(t0 + kTile);
        if (t0 + kTile <= L && t0 + kTile - 1 <= pos_min)
            score_tile(t0, std::false_type{});
        else
            score_tile(t0, std::true_type{});
        __syncthreads();
        // rows of 64 block scores per query, with non-temporal stores (the
        // writes are as many bytes as the index reads at Q = 64, and ordinary
        // stores slow the read stream down)
        const int blk0 = t0 / kBT;
#pragma unroll
        for (int k = 0; k < Q / 4; k++) {
            const int idx = tid + kThreads * k;
            const int qi = idx >> 6;
            const int blk = blk0 + (idx & 63);
            if (blk < n_blk)
                __builtin_nontemporal_store(stage[qi][(idx & 63) ^ (16 * (qi & 1))],
                                            out_b + (int64_t)qi * bs_stride + blk);
        }
    }
}

} // namespace

hipError_t launch_multi_score(int n_queries, const uint8_t *keys, const uint16_t *scales, const uint16_t *q_idx,
                              const float *w_idx, const int32_t *q_pos, const int32_t *ctx_len, const int64_t *row0,
                              int64_t n_rows, int batch, int max_ctx, float *out, int64_t bs_stride, hipStream_t s)
{
    if (max_ctx <= 0)
        return hipSuccess;
    int chunk = kTile;
    while (chunk < 4096 && (int64_t)batch * ((max_ctx + 2 * chunk - 1) / (2 * chunk)) >= 1024)
        chunk *= 2;
    dim3 grid((unsigned)((max_ctx + chunk - 1) / chunk), (unsigned)batch);
#define QSA_MULTI(RB)                                                                                          \
    hipLaunchKernelGGL((multi_score_kernel<RB>), grid, dim3(kThreads), 0, s, keys, scales, q_idx, w_idx, q_pos, \
                       ctx_len, row0, n_rows, max_ctx, chunk, out, bs_stride)
    switch (n_queries / 4) {
    case 1: QSA_MULTI(1); break;
    case 2: QSA_MULTI(2); break;
    case 4: QSA_MULTI(4); break;
    case 8: QSA_MULTI(8); break;
    case 16: QSA_MULTI(16); break;
    default: return hipErrorInvalidValue;
    }
#undef QSA_MULTI
    return hipGetLastError();
}

} // namespace qsa
