/*
 * synth_host.c -- host C version of the seeded input generator (inputs only).
 *
 * Produces exactly the bytes of the numpy generator in qsa_synth/__init__.py
 * (index keys with their per-token e4m3 quantisation, and bf16 KV rows), only
 * faster, so that large samples can be regenerated on the CPU. It holds none
 * of the method's arithmetic. Built with gcc -ffp-contract=off on x86-64, where
 * float arithmetic is IEEE single precision, like numpy's float32.
 *
 * Generator: SplitMix64 in counter mode (Steele, Lea and Flood, OOPSLA 2014);
 * normals are Irwin-Hall sums of twelve 16-bit uniforms, centred and scaled by
 * 2^-16 (an integer computation, exact in float).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static const uint64_t kGamma = 0x9E3779B97F4A7C15ull;

static uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint64_t tensor, uint64_t layer)
{
    return mix64((seed << 32) ^ (tensor << 16) ^ layer);
}

static float normal_at(uint64_t key, uint64_t n)
{
    int64_t acc = 0;
    for (int j = 0; j < 3; j++) {
        uint64_t o = mix64(key + (3 * n + (uint64_t)j + 1) * kGamma);
        acc += (int64_t)(o & 0xFFFF) + (int64_t)((o >> 16) & 0xFFFF) + (int64_t)((o >> 32) & 0xFFFF) +
               (int64_t)(o >> 48);
    }
    return (float)(int)(acc - 393210) * (1.0f / 65536.0f);
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float bits_f32(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* IEEE binary32 -> binary16, round to nearest even (finite, non-negative use). */
uint16_t synth_f32_to_f16(float f)
{
    uint32_t u = f32_bits(f);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return (uint16_t)(sign | 0x7E00u);
    if (a >= 0x477FF000u)                   /* >= 65520 rounds to infinity */
        return (uint16_t)(sign | 0x7C00u);
    if (a >= 0x38800000u) {                 /* normal half: >= 2^-14 */
        uint32_t r = (a + 0xFFFu + ((a >> 13) & 1u)) >> 13;
        return (uint16_t)(sign | (r - (112u << 10)));
    }
    /* subnormal half: m * 2^-24, m = rint(x * 2^24) (exact scaling) */
    return (uint16_t)(sign | (uint32_t)rintf(bits_f32(a) * 16777216.0f));
}

static float f16_to_f32(uint16_t h)
{
    uint32_t e = (h >> 10) & 31u, m = h & 1023u;
    float mag = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(1024u + m), (int)e - 25);
    return (h & 0x8000u) ? -mag : mag;
}

static uint16_t bf16_rne(float x)
{
    uint32_t u = f32_bits(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static uint8_t e4m3_rne_sat(float x)
{
    uint32_t u = f32_bits(x);
    uint32_t sign = (u >> 31) << 7;
    uint32_t a = u & 0x7FFFFFFFu;
    float af = bits_f32(a);
    int code;
    if (af >= 448.0f) {
        code = 0x7E;
    } else if ((int)(a >> 23) - 127 >= -6) {
        code = (int)((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120 << 3);
        if (code > 0x7E)
            code = 0x7E;
    } else {
        code = (int)rintf(af * 512.0f);
    }
    return (uint8_t)((uint32_t)code | sign);
}

static int is_planted(const int32_t *planted, int n_planted, int32_t blk)
{
    int lo = 0, hi = n_planted;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (planted[mid] < blk)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo < n_planted && planted[lo] == blk;
}

/* Quantised index keys of tokens [t0, t1) of sequence b in one layer:
 * codes[(t - t0) * 64 + i], sig[t - t0]. planted: sorted block list; u: float[64]. */
void synth_index_keys(uint64_t seed, int layer, int b, int64_t t0, int64_t t1, const int32_t *planted,
                      int n_planted, const float *u, int block_tokens, uint8_t *codes, uint16_t *sig)
{
    uint64_t km = stream_key(seed, 4, (uint64_t)layer);
    uint64_t kn = stream_key(seed, 5, (uint64_t)layer);
    for (int64_t t = t0; t < t1; t++) {
        int hit = is_planted(planted, n_planted, (int32_t)(t / block_tokens));
        uint64_t base = (((uint64_t)b << 28) + (uint64_t)t) * 64u;
        float x[64];
        float amax = 0.0f;
        for (int i = 0; i < 64; i++) {
            float v;
            if (hit) {
                float noise = normal_at(kn, base + (uint64_t)i);
                float scaled = 0.1f * noise;
                v = u[i] + scaled;
            } else {
                v = normal_at(km, base + (uint64_t)i);
            }
            x[i] = v;
            float av = fabsf(v);
            amax = av > amax ? av : amax;
        }
        float q = amax / 448.0f;
        uint16_t s16 = synth_f32_to_f16(q);
        float s32 = f16_to_f32(s16);
        uint8_t *dst = codes + (t - t0) * 64;
        for (int i = 0; i < 64; i++)
            dst[i] = s32 > 0.0f ? e4m3_rne_sat(x[i] / s32) : 0;
        sig[t - t0] = s16;
    }
}

/* bf16 rows [n][row_elems] of the given physical slots of one layer's pool. */
void synth_kv_rows(uint64_t seed, int layer, const int64_t *slots, int64_t n, int64_t row_elems, uint16_t *out)
{
    uint64_t key = stream_key(seed, 6, (uint64_t)layer);
    for (int64_t r = 0; r < n; r++) {
        uint64_t n0 = (uint64_t)slots[r] * (uint64_t)row_elems;
        for (int64_t e = 0; e < row_elems; e++)
            out[r * row_elems + e] = bf16_rne(normal_at(key, n0 + (uint64_t)e));
    }
}
