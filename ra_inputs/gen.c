/*
 * Seeded synthetic inputs for the attention tests and the benchmark.
 *
 * This module is shared by the CPU oracle side and the GPU side, and by
 * design it holds none of the attention arithmetic: only
 *   - the Philox4x32-10 counter-based generator (J. K. Salmon, M. A. Moraes,
 *     R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
 *     SC'11), written from the paper's definition;
 *   - the Box-Muller transform (G. E. P. Box, M. E. Muller, 1958) that turns
 *     two uniforms into two N(0,1) deviates;
 *   - round-to-nearest-even narrowing of binary32 to bfloat16.
 *
 * Value of element (b, h, t, k) of a [B, H, S, d] tensor drawn from stream
 * (seed, stream_id) is a pure function of its flat index
 *     i = ((b*H + h)*S + t)*d + k,
 * so any shard (a contiguous chunk, a striped subset of tokens, one head) is
 * produced without generating the whole tensor.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC gen.c -o libra_inputs.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

/* One Philox4x32 bijection round: two 32x32->64 multiplies, xor with key. */
static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

/* Philox4x32 with 10 rounds; the key is bumped by the Weyl constants between
 * rounds. Exported so tests can check the published known-answer vectors. */
void rin_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k[0] += PHILOX_W0;
            k[1] += PHILOX_W1;
        }
        philox_round(c, k);
    }
    memcpy(out, c, sizeof(c));
}

/* Four N(0,1) deviates (as binary32) for Philox block number g of a stream. */
static void normal4(uint64_t seed, uint32_t stream_id, uint64_t g, float z[4]) {
    const uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), stream_id, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t x[4];
    rin_philox4x32_10(ctr, key, x);
    const double two_m32 = 2.3283064365386963e-10; /* 2^-32 */
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double u1 = ((double)x[2 * p] + 1.0) * two_m32; /* (0, 1] */
        double u2 = (double)x[2 * p + 1] * two_m32;     /* [0, 1) */
        double r = sqrt(-2.0 * log(u1));
        z[2 * p] = (float)(r * cos(two_pi * u2));
        z[2 * p + 1] = (float)(r * sin(two_pi * u2));
    }
}

/* binary32 -> bfloat16 bits, round to nearest, ties to even (finite input). */
uint16_t rin_f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) /* inf / nan: truncate, keep quiet bit */
        return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/*
 * Fill out[B, H, n_rows, d] with scale * N(0,1) values of the logical tensor
 * [B, H, S, d] drawn from stream (seed, stream_id), taking token rows
 * t = t0 + r * t_stride for r in [0, n_rows).  t may fall outside [0, S): the
 * flat index is then taken modulo 2^64, which is still a valid counter.
 * out_dtype: 0 = binary32, 1 = bfloat16 bits (round to nearest even of the
 * scaled binary32 value).  Returns 0, or -1 on a bad argument.
 */
int rin_normal_rows(uint64_t seed, uint32_t stream_id, int64_t B, int64_t H, int64_t S,
                    int64_t d, int64_t t0, int64_t t_stride, int64_t n_rows, int out_dtype,
                    float scale, void* out) {
    if (B < 0 || H < 0 || S < 0 || d <= 0 || n_rows < 0 || !out) return -1;
    if (out_dtype != 0 && out_dtype != 1) return -1;
    const int64_t total_rows = B * H * n_rows;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < total_rows; ++row) {
        const int64_t r = row % n_rows;
        const int64_t bh = row / n_rows;
        const int64_t t = t0 + r * t_stride;
        const uint64_t base = (uint64_t)((bh * S + t) * d);
        float zbuf[4];
        uint64_t cached = UINT64_MAX;
        for (int64_t k = 0; k < d; ++k) {
            const uint64_t i = base + (uint64_t)k;
            const uint64_t g = i >> 2;
            if (g != cached) {
                normal4(seed, stream_id, g, zbuf);
                cached = g;
            }
            const float v = scale * zbuf[i & 3u];
            if (out_dtype == 0)
                ((float*)out)[row * d + k] = v;
            else
                ((uint16_t*)out)[row * d + k] = rin_f32_to_bf16_rne(v);
        }
    }
    return 0;
}

/* Widen bfloat16 bits to binary32 (exact). */
void rin_bf16_to_f32(const uint16_t* x, float* y, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)x[i] << 16;
        memcpy(&y[i], &u, 4);
    }
}
