// bench_stream.hip -- the streaming-read reference that bench.py measures
// beside the decode step: how fast this GPU reads a large device buffer
// front to back, so that the step's and the index scan's achieved GB/s can
// be given as fractions of a ceiling measured on the same machine, next to the
// published HBM peak. Not part of libqsa.
//
// Workgroup w (256 threads) reads bytes [w * chunk, (w + 1) * chunk) of buf,
// each lane keeping eight 16-byte non-temporal loads in flight, and folds
// them into one word per thread (so that the loads are not removed). chunk
// must be a multiple of 256 * 16 * 8 bytes; the grid covers n_wg chunks, all
// inside buf.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ buf, int64_t chunk_vec,
                                                          uint32_t *__restrict__ out)
{
    const int64_t base = (int64_t)blockIdx.x * chunk_vec;
    uint32_t acc = 0;
    for (int64_t i = threadIdx.x; i < chunk_vec; i += 256 * 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; u++)
            v[u] = __builtin_nontemporal_load(buf + base + i + u * 256);
#pragma unroll
        for (int u = 0; u < 8; u++)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

extern "C" int bench_stream_read(const void *buf, int64_t n_wg, int64_t chunk_bytes, uint32_t *out, hipStream_t s)
{
    if (!buf || !out || n_wg <= 0 || n_wg > INT32_MAX || chunk_bytes <= 0 || chunk_bytes % (256 * 16 * 8) != 0)
        return 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)n_wg), dim3(256), 0, s, (const u32x4 *)buf,
                       chunk_bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
