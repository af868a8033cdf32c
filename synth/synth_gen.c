/*
 * Seeded synthetic inputs: counter-based normal draws rounded to fp32 or bf16.
 *
 * This file holds no attention arithmetic. It produces the host buffers that
 * both the GPU path and the fp64 oracle read, so the two sides see identical
 * data without sharing any code of the method.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), written from its published
 * definition: 10 rounds of two 32x32->64 multiplies (multipliers 0xD2511F53
 * and 0xCD9E8D57) with a Weyl key schedule (0x9E3779B9, 0xBB67AE85).
 *
 * Element e (row-major flat index of the full tensor) takes counter
 * {e/4 low, e/4 high, tensor_id, 0} and key {seed low, seed high}; the block's
 * four words feed two Box-Muller pairs (x0,x1) and (x2,x3), and element e gets
 * the (e mod 4)-th normal. Each uniform is (x + 0.5) * 2^-32, in (0, 1).
 * Any element can therefore be regenerated on its own.
 *
 * Rounding: the fp64 normal times the caller's factor is rounded to fp32 by
 * round-to-nearest-even (a C cast), then to bf16 by round-to-nearest-even on
 * the fp32 bit pattern.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t x[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * x[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * x[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t y0 = hi1 ^ x[1] ^ k[0];
    uint32_t y2 = hi0 ^ x[3] ^ k[1];
    x[0] = y0;
    x[1] = lo1;
    x[2] = y2;
    x[3] = lo0;
}

/* Philox4x32-10: ctr and key in, 4 words out (in place in ctr). */
void synth_philox4x32_10(uint32_t ctr[4], const uint32_t key_in[2]) {
    uint32_t k[2] = {key_in[0], key_in[1]};
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k[0] += PHILOX_W0;
            k[1] += PHILOX_W1;
        }
        philox_round(ctr, k);
    }
}

static inline void block_words(uint64_t seed, uint32_t tensor_id, uint64_t blk, uint32_t out[4]) {
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    out[0] = (uint32_t)blk;
    out[1] = (uint32_t)(blk >> 32);
    out[2] = tensor_id;
    out[3] = 0;
    synth_philox4x32_10(out, key);
}

/* Raw words: n consecutive 32-bit outputs of the stream (seed, tensor_id),
 * word w = output (w mod 4) of block w/4. */
void synth_raw_u32(uint64_t seed, uint32_t tensor_id, uint64_t first, uint64_t n, uint32_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint64_t w = first + (uint64_t)i;
        uint32_t b[4];
        block_words(seed, tensor_id, w >> 2, b);
        out[i] = b[w & 3];
    }
}

static inline double u01(uint32_t x) { return ((double)x + 0.5) * (1.0 / 4294967296.0); }

/* The four fp64 N(0,1) draws of one block. */
static inline void block_normals(uint64_t seed, uint32_t tensor_id, uint64_t blk, double z[4]) {
    uint32_t b[4];
    block_words(seed, tensor_id, blk, b);
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double r = sqrt(-2.0 * log(u01(b[2 * p])));
        double t = two_pi * u01(b[2 * p + 1]);
        z[2 * p] = r * cos(t);
        z[2 * p + 1] = r * sin(t);
    }
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) /* NaN: keep it quiet */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)((u + bias) >> 16);
}

uint16_t synth_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/*
 * Fill rows [row_lo, row_hi) of every (b, h) of a [B, H, S, D] tensor whose
 * full extent is S rows. out is [B, H, row_hi-row_lo, D] contiguous.
 * value = factor * (row_factor ? row_factor[s] : 1) * z, in fp64, then rounded.
 * out_kind: 0 = fp64, 1 = fp32, 2 = bf16 (uint16 bit patterns).
 */
int synth_normal_rows(uint64_t seed, uint32_t tensor_id, int64_t B, int64_t H, int64_t S, int64_t D,
                      int64_t row_lo, int64_t row_hi, double factor, const double* row_factor,
                      int out_kind, void* out) {
    if (B < 0 || H < 0 || S < 0 || D <= 0 || row_lo < 0 || row_hi < row_lo || row_hi > S) return -1;
    if (out_kind < 0 || out_kind > 2) return -2;
    const int64_t R = row_hi - row_lo;
    const int64_t nrows = B * H * R;
    #pragma omp parallel for schedule(static)
    for (int64_t rr = 0; rr < nrows; ++rr) {
        int64_t bh = rr / R, s = row_lo + rr % R;
        double f = factor * (row_factor ? row_factor[s] : 1.0);
        uint64_t e0 = (uint64_t)((bh * S + s) * D);
        double z[4];
        uint64_t cur_blk = UINT64_MAX;
        for (int64_t d = 0; d < D; ++d) {
            uint64_t e = e0 + (uint64_t)d;
            if ((e >> 2) != cur_blk) {
                cur_blk = e >> 2;
                block_normals(seed, tensor_id, cur_blk, z);
            }
            double x = f * z[e & 3];
            int64_t o = rr * D + d;
            if (out_kind == 0) {
                ((double*)out)[o] = x;
            } else {
                float xf = (float)x;
                if (out_kind == 1) ((float*)out)[o] = xf;
                else ((uint16_t*)out)[o] = f32_to_bf16_rne(xf);
            }
        }
    }
    return 0;
}
