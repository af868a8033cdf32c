/*
 * ORACLE — test infrastructure only.  Plain, slow, fp64 softmax attention on
 * the CPU.  Only the tests, the smoke check and the bench's CPU-baseline leg
 * may load this library; the GPU path never does.  It shares no code with the
 * GPU path: inputs arrive as host buffers and are widened here, exactly, to
 * fp64.
 *
 * What it computes is the textbook definition of bidirectional (non-causal)
 * multi-head softmax attention, which the blockwise online-softmax method
 * reaches exactly up to rounding (NVIDIA Technical Blog "Scaling AI Inference
 * Across Multiple GPUs Using NVIDIA TensorRT with Multi-Device Inference
 * Support": section "Context parallelism" — DiT attention is bidirectional;
 * section "AllGather KV" — each rank's query slice attends over the full
 * sequence; section "Ring Attention" — with an online softmax the full K and
 * V never need to be materialised, so blockwise evaluation gives the same
 * result; section "DeepSpeed Ulysses" — full-sequence attention on a subset
 * of heads).  The pages print no formula; the one used is, for query row i
 * of head (b, h) and every key j in the chosen key range:
 *
 *     s_ij = scale * sum_d Q[i,d] K[j,d]
 *     m_i  = max_j s_ij
 *     w_ij = exp(s_ij - m_i),  l_i = sum_j w_ij,  P_ij = w_ij / l_i
 *     O[i,:] = sum_j P_ij V[j,:]
 *     LSE_i  = m_i + ln l_i                     (natural log, scale included)
 *
 * An empty key range gives O = 0 and LSE = -inf.
 *
 * The merge below combines results over disjoint key ranges; it follows from
 * the definition: with M = max_c LSE_c, LSE = M + ln sum_c exp(LSE_c - M) and
 * O = sum_c exp(LSE_c - LSE) O_c.  Parts with LSE_c = -inf carry no weight.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { K_F64 = 0, K_F32 = 1, K_BF16 = 2 };

/* Exact widening of one stored element to fp64. */
static inline double widen(const void* base, int kind, int64_t i) {
    if (kind == K_F64) return ((const double*)base)[i];
    if (kind == K_F32) return (double)((const float*)base)[i];
    uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Attention of R query rows per (b, h) against keys [kv_lo, kv_hi).
 *   q: [B, H, R, D]; k, v: [B, H, Skv, D]; all contiguous, element kinds as above.
 *   o: [B, H, R, D] fp64; lse: [B, H, R] fp64; p (optional, may be NULL):
 *   [B, H, R, kv_hi - kv_lo] fp64 softmax probabilities.
 * Returns 0, or a negative value for inconsistent arguments.
 */
int oracle_attention(int64_t B, int64_t H, int64_t R, int64_t Skv, int64_t D, double scale,
                     const void* q, int q_kind, const void* k, int k_kind, const void* v, int v_kind,
                     int64_t kv_lo, int64_t kv_hi, double* o, double* lse, double* p, int nthreads) {
    if (B < 0 || H < 0 || R < 0 || Skv < 0 || D <= 0) return -1;
    if (kv_lo < 0 || kv_hi < kv_lo || kv_hi > Skv) return -2;
    const int64_t n = kv_hi - kv_lo;
    const int64_t rows = B * H * R;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    #pragma omp parallel
    {
        double* s = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t row = 0; row < rows; ++row) {
            const int64_t bh = row / R;
            const int64_t q0 = row * D;
            double* orow = o + row * D;
            if (n == 0) {
                for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
                lse[row] = -INFINITY;
                continue;
            }
            /* scores */
            for (int64_t j = 0; j < n; ++j) {
                const int64_t k0 = (bh * Skv + kv_lo + j) * D;
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d) acc += widen(q, q_kind, q0 + d) * widen(k, k_kind, k0 + d);
                s[j] = scale * acc;
            }
            /* exact max, exponentials, normaliser */
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j)
                if (s[j] > m) m = s[j];
            double l = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            /* probabilities and weighted sum of V rows */
            for (int64_t j = 0; j < n; ++j) s[j] = s[j] / l;
            if (p)
                for (int64_t j = 0; j < n; ++j) p[row * n + j] = s[j];
            for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const int64_t v0 = (bh * Skv + kv_lo + j) * D;
                for (int64_t d = 0; d < D; ++d) orow[d] += s[j] * widen(v, v_kind, v0 + d);
            }
            lse[row] = m + log(l);
        }
        free(s);
    }
    return 0;
}

/*
 * Merge n results over disjoint key ranges, row by row.
 *   o_parts[c]: [rows, D] fp64; lse_parts[c]: [rows] fp64; o: [rows, D]; lse: [rows].
 */
int oracle_lse_merge(int64_t n, int64_t rows, int64_t D, const double* const* o_parts,
                     const double* const* lse_parts, double* o, double* lse) {
    if (n < 1 || rows < 0 || D <= 0) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int64_t c = 0; c < n; ++c)
            if (lse_parts[c][r] > M) M = lse_parts[c][r];
        double* orow = o + r * D;
        for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
        if (M == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double ssum = 0.0;
        for (int64_t c = 0; c < n; ++c) ssum += exp(lse_parts[c][r] - M);
        const double L = M + log(ssum);
        for (int64_t c = 0; c < n; ++c) {
            const double w = exp(lse_parts[c][r] - L);
            for (int64_t d = 0; d < D; ++d) orow[d] += w * o_parts[c][r * D + d];
        }
        lse[r] = L;
    }
    return 0;
}
