// append.hip -- the append step: the decode step's new token enters the
// cache of every QSA layer.
//
// For sequence b with current length t = ctx_len[b] and the slot s the caller
// allocated for the token, every layer l gets
//   - index row idx_row0[b] + t: the new index key quantised to e4m3 with one
//     fp16 scale (sigma = fp16(amax / 448), code_i = e4m3(x_i / sigma), both
//     divisions in binary32, round to nearest even, magnitudes clamped to 448);
//   - KV pool row s: the token's K and V row, copied as is;
// then the page table maps t -> s and the length becomes t + 1 (article,
// memory-ledger section: the index, its quantisation scales and the page
// layout are kept aligned, and logical token addresses are mapped to physical
// cache slots).
//
// One wave per sequence walks the layers: lane i quantises element i of the
// 64-element key and copies 32 bytes of the 2 KB row. The sequence's length
// is read once, before anything is written, so the length may be updated in
// place.
#include "qsa_internal.h"

#include <hip/hip_fp16.h>

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
constexpr int kAppendGroup = 12;

// binary32 -> OCP e4m3 code, round to nearest even, |y| >= 448 clamped to 448.
__device__ __forceinline__ uint32_t e4m3_of(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x43E00000u)                      // 448.0f and above
        return sign | 0x7Eu;
    if (a < 0x3C800000u)                       // below 2^-6: multiples of 2^-9
        return sign | (uint32_t)rintf(__uint_as_float(a) * 512.0f);
    // keep 3 of 23 mantissa bits (nearest even), then rebias 127 -> 7
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    const uint32_t code = r - (120u << 3);
    return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__global__ __launch_bounds__(64) void append_kernel(AppendLayers ly, int n_layers, const int32_t *__restrict__ ctx_len,
                                                    const int64_t *__restrict__ row0, int64_t n_rows,
                                                    int64_t pt_stride, int64_t n_slots,
                                                    const int32_t *__restrict__ new_slot,
                                                    int32_t *__restrict__ page_table, int32_t *__restrict__ ctx_out,
                                                    const uint32_t *__restrict__ new_gen,
                                                    uint32_t *__restrict__ tok_gen)
{
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int t = ctx_len[b];
    const int64_t r0 = row0[b];
    const int32_t slot = new_slot[b];
    const bool ok = t >= 0 && (int64_t)t < pt_stride && r0 >= 0 && r0 + t < n_rows && slot >= 0 &&
                    (int64_t)slot < n_slots;
    if (ok) {
        const int64_t row = r0 + t;
        // Layers in groups of kAppendGroup: every load of a group is issued
        // before the first store, so a group costs one memory round trip.
        for (int l0 = 0; l0 < n_layers; l0 += kAppendGroup) {
            float x[kAppendGroup];
            u32x4 v0[kAppendGroup], v1[kAppendGroup];
#pragma unroll
            for (int j = 0; j < kAppendGroup; j++) {
                const int l = l0 + j;
                if (l < n_layers) {
                    x[j] = ly.new_key[l][(int64_t)b * kIdxD + lane];
                    const u32x4 *src = reinterpret_cast<const u32x4 *>(ly.new_row[l] + (int64_t)b * kRowBytes);
                    v0[j] = src[lane];
                    v1[j] = src[lane + 64];
                }
            }
#pragma unroll
            for (int j = 0; j < kAppendGroup; j++) {
                const int l = l0 + j;
                if (l >= n_layers)
                    break;
                float amax = fabsf(x[j]);
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1)
                    amax = fmaxf(amax, __shfl_xor(amax, o));
                const __half s16 = __float2half_rn(amax / 448.0f);
                const float sigma = __half2float(s16);
                const uint32_t code = sigma > 0.0f ? e4m3_of(x[j] / sigma) : 0u;
                ly.keys[l][row * kIdxD + lane] = (uint8_t)code;
                if (lane == 0)
                    ly.scales[l][row] = __half_as_ushort(s16);
                u32x4 *dst = reinterpret_cast<u32x4 *>(ly.pool[l] + (int64_t)slot * kRowBytes);
                dst[lane] = v0[j];
                dst[lane + 64] = v1[j];
            }
        }
    }
    if (lane == 0) {
        if (ok) {
            page_table[(int64_t)b * pt_stride + t] = slot;
            if (tok_gen)
                tok_gen[(int64_t)b * pt_stride + t] = new_gen ? new_gen[b] : 0u;
        }
        if (ctx_out)
            ctx_out[b] = ok ? t + 1 : t;
    }
}

} // namespace

hipError_t launch_append(const AppendLayers &ly, int n_layers, int batch, const int32_t *ctx_len,
                         const int64_t *row0, int64_t n_rows, int64_t pt_stride, int64_t n_slots,
                         const int32_t *new_slot, int32_t *page_table, int32_t *ctx_out, const uint32_t *new_gen,
                         uint32_t *tok_gen, hipStream_t s)
{
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)batch), dim3(64), 0, s, ly, n_layers, ctx_len, row0, n_rows,
                       pt_stride, n_slots, new_slot, page_table, ctx_out, new_gen, tok_gen);
    return hipGetLastError();
}

} // namespace qsa
