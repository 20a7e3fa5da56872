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

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int kWaveTok = 64;
constexpr int kWgTok = kThreads / 64 * kWaveTok;   // 256

template <int RB>
__global__ __launch_bounds__(kThreads) void multi_score_kernel(
    const uint8_t *__restrict__ keys, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ q_idx,
    const float *__restrict__ w_idx, const int32_t *__restrict__ q_pos, const int32_t *__restrict__ ctx_len,
    const int64_t *__restrict__ row0, int64_t n_rows, int max_ctx, int chunk_tokens, float *__restrict__ out,
    int64_t bs_stride)
{
    constexpr int Q = 4 * RB;
    __shared__ float wq[Q][kIdxH];
    __shared__ int32_t posq[Q];

    const int b = blockIdx.y;
    const int64_t r0 = row0[b];
    int L = clamp_ctx(ctx_len[b], max_ctx);
    if (r0 < 0 || r0 + L > n_rows)
        L = 0;
    const int t_begin = blockIdx.x * chunk_tokens;
    if (t_begin >= L)
        return;
    const int n_blk = (L + kBT - 1) / kBT;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint8_t *kbase = keys + r0 * kIdxD;
    const uint16_t *sbase = scales + r0;
    const int t_end = min(t_begin + chunk_tokens, L);

    u32x4 k[4], kn[4];
    uint16_t sc_bits = 0, sc_next = 0;
    const int grp_tok = lane & 15;
    const int grp_off = 16 * (lane >> 4);
    auto load_tile = [&](int tw, u32x4 *dst, uint16_t &sc) {
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int t = tw + 16 * g + grp_tok;
            dst[g] = t < L ? __builtin_nontemporal_load(
                                 reinterpret_cast<const u32x4 *>(kbase + (int64_t)t * kIdxD + grp_off))
                           : u32x4{0u, 0u, 0u, 0u};
        }
        sc = (tw + lane < L) ? sbase[tw + lane] : (uint16_t)0;
    };
    int tw = t_begin + wave * kWaveTok;
    if (tw < t_end)
        load_tile(tw, k, sc_bits);

    if (tid < Q * kIdxH)
        wq[tid / kIdxH][tid % kIdxH] = w_idx[((int64_t)b * Q) * kIdxH + tid];
    if (tid < Q)
        posq[tid] = q_pos[(int64_t)b * Q + tid];
    // A operands: row block r, lane l: row l & 15 = query 4 r + ((l & 15) >> 2),
    // head (l & 3); dims follow the lane's key bytes (16 (l >> 4) + 0..7 for
    // the first MFMA, + 8..15 for the second).
    bf16x8 qa[RB][2];
#pragma unroll
    for (int r = 0; r < RB; r++) {
        const int qi = 4 * r + ((lane & 15) >> 2);
        const u32x4 *qrow = reinterpret_cast<const u32x4 *>(
            q_idx + (((int64_t)b * Q + qi) * kIdxH + (lane & 3)) * kIdxD + 16 * (lane >> 4));
        qa[r][0] = __builtin_bit_cast(bf16x8, qrow[0]);
        qa[r][1] = __builtin_bit_cast(bf16x8, qrow[1]);
    }
    __syncthreads();

    float *out_b = out + (int64_t)b * Q * bs_stride;
    for (; tw < t_end; tw += kWgTok) {
        const int tn = tw + kWgTok;
        if (tn < t_end)
            load_tile(tn, kn, sc_next);
        const float sig_lane = (float)__builtin_bit_cast(_Float16, sc_bits);
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const bf16x8 kb0 = e4m3x8_to_bf16x8(k[g].x, k[g].y);
            const bf16x8 kb1 = e4m3x8_to_bf16x8(k[g].z, k[g].w);
            const int t = tw + 16 * g + (lane & 15);
            const float sigma = __shfl(sig_lane, 16 * g + (lane & 15));
            const int blk = t >> 2;
#pragma unroll
            for (int r = 0; r < RB; r++) {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[r][0], kb0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[r][1], kb1, acc, 0, 0, 0);
                // acc[h] = q_{4r + (l>>4), h} . k_t
                const int qi = 4 * r + (lane >> 4);
                float s = -INFINITY;
                if (t < L && t <= posq[qi]) {
                    s = 0.0f;
                    s += wq[qi][0] * fmaxf(sigma * acc[0], 0.0f);
                    s += wq[qi][1] * fmaxf(sigma * acc[1], 0.0f);
                    s += wq[qi][2] * fmaxf(sigma * acc[2], 0.0f);
                    s += wq[qi][3] * fmaxf(sigma * acc[3], 0.0f);
                }
                s = fmaxf(s, __shfl_xor(s, 1));
                s = fmaxf(s, __shfl_xor(s, 2));
                if ((lane & 3) == 0 && blk < n_blk)
                    out_b[(int64_t)qi * bs_stride + blk] = s;
            }
        }
#pragma unroll
        for (int g = 0; g < 4; g++)
            k[g] = kn[g];
        sc_bits = sc_next;
    }
}

} // namespace

hipError_t launch_multi_score(int n_queries, const uint8_t *keys, const uint16_t *scales, const uint16_t *q_idx,
                              const float *w_idx, const int32_t *q_pos, const int32_t *ctx_len, const int64_t *row0,
                              int64_t n_rows, int batch, int max_ctx, float *out, int64_t bs_stride, hipStream_t s)
{
    if (max_ctx <= 0)
        return hipSuccess;
    int chunk = kWgTok;
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
