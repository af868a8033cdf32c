// Log-sum-exp merge of per-chunk attention results, the merge of the stream-K tail's partials,
// and the empty-chunk fill.
//
// Results over disjoint key sets combine exactly: with M = max_c LSE_c,
//   LSE = M + ln sum_c exp(LSE_c - M),   O = sum_c exp(LSE_c - LSE) O_c.
// This is the online-softmax update that folds each arriving key/value block
// into a rank's attention output (NVIDIA Technical Blog "Scaling AI
// Inference Across Multiple GPUs Using NVIDIA TensorRT with Multi-Device
// Inference Support", section "Ring Attention"), applied to n blocks at once.
//
// The merge streams n fp32 partials and writes one output: it is bound by
// HBM bandwidth.  Each lane owns 4 consecutive elements of a row (16-byte
// loads), a row's D/4 lanes sit in one wave, and every part is read exactly
// once.  Parts are taken in batches (2 to 16 parts, the smallest that covers
// n, up to 16) with all of a batch's loads issued before any is used, so each
// lane keeps a batch of loads in flight.  The parts are read, and the output written, once:
// non-temporal accesses keep them from displacing other data in the caches (measured 5.4 ->
// 5.8 TB/s for 8 parts of 44,160 x 16 rows).
// Parts whose LSE is -inf carry no weight; if all are -inf the output is
// O = 0, LSE = -inf.
#include "kernels.h"

#include <math.h>

namespace lsdit {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ void store4(void* o, Strides os, int o_bf16, int H, int Sq, int64_t row, int d, f32x4_t x) {
    const int64_t bh = row / Sq, s = row % Sq;
    const int64_t b = bh / H, h = bh % H;
    const int64_t off = b * os.b + h * os.h + s * os.s + d;
    if (o_bf16) {
        u32x2_t w;
        w[0] = pack_bf16(x[0], x[1]);
        w[1] = pack_bf16(x[2], x[3]);
        __builtin_nontemporal_store(w, (u32x2_t*)((unsigned short*)o + off));
    } else {
        __builtin_nontemporal_store(x, (f32x4_t*)((float*)o + off));
    }
}

template <int kBatch>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
    const int lanes_per_row = a.D / 4;
    const int rows_per_block = kThreads / lanes_per_row;
    const int64_t rows = (int64_t)a.B * a.H * a.Sq;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / lanes_per_row;
    const int d = 4 * (threadIdx.x % lanes_per_row);
    if (row >= rows) return;
    const int n = a.n;

    // LSE of the union, natural-log domain (so that a single live part gets weight
    // exp(0) = 1 and passes through exactly): running max M and sum of exp(LSE_c - M)
    float M = -INFINITY, tot = 0.f;
    for (int c0 = 0; c0 < n; c0 += kBatch) {
        float l[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) l[u] = c0 + u < n ? a.lse_parts[c0 + u][row] : -INFINITY;
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) mb = fmaxf(mb, l[u]);
        if (mb == -INFINITY) continue;  // nothing live in this batch
        const float m_new = fmaxf(M, mb);
        float sb = 0.f;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) sb += expf(l[u] - m_new);
        tot = (M == -INFINITY ? 0.f : tot * expf(M - m_new)) + sb;
        M = m_new;
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float lse_out = -INFINITY;
    if (M != -INFINITY) {
        const float L = M + logf(tot);
        for (int c0 = 0; c0 < n; c0 += kBatch) {
            f32x4_t x[kBatch];
            float w[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const bool live = c0 + u < n;
                x[u] = live ? __builtin_nontemporal_load((const f32x4_t*)(a.o_parts[c0 + u] + row * a.D + d))
                            : f32x4_t{0.f, 0.f, 0.f, 0.f};
                w[u] = live ? a.lse_parts[c0 + u][row] : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) acc += expf(w[u] - L) * x[u];
        }
        lse_out = L;
    }
    store4(a.o, a.os, a.o_bf16, a.H, a.Sq, row, d, acc);
    // lse_parts[0] may alias lse: this store depends on every load of it above.
    if (d == 0) a.lse[row] = lse_out;
}

// The stream-K tail of the bf16 kernel (FwdArgs) left, for each query tile j of the tail, fp32
// partials over consecutive runs of its T key tiles in the slots of the workgroups whose unit
// ranges meet [jT, (j+1)T).  The first of them is the last workgroup starting at or before jT:
// w = floor(((jT + 1) P - 1) / U) for P workgroups over U units (ranges may be empty when U < P).
// A run that starts before jT is its workgroup's second segment.  The runs merge by the LSE rule
// above; a tile's rows are read and written once.
__global__ __launch_bounds__(kThreads) void sk_fixup_kernel(SkFixupArgs a) {
    const int lanes_per_row = a.D / 4;
    const int rows_per_block = kThreads / lanes_per_row;
    const int blocks_per_tile = kSkRows / rows_per_block;
    const int j = blockIdx.x / blocks_per_tile;
    const int r = (blockIdx.x % blocks_per_tile) * rows_per_block + threadIdx.x / lanes_per_row;
    const int d = 4 * (threadIdx.x % lanes_per_row);
    const int tile = a.n_dp + j;
    const int bh = tile / a.n_qt, s = (tile % a.n_qt) * kSkRows + r;
    if (s >= a.Sq) return;
    const int P = a.sk_wgs;
    const int64_t U = (int64_t)(a.n_q - a.n_dp) * a.T;
    const int64_t t0 = (int64_t)j * a.T, t1 = t0 + a.T;
    const int w0 = (int)(((t0 + 1) * P - 1) / U);

    float M = -INFINITY, tot = 0.f;
    for (int w = w0; w < P; ++w) {
        const int64_t u0 = sk_start(U, w, P), u1 = sk_start(U, w + 1, P);
        if (u0 >= t1) break;
        if (u1 == u0) continue;
        const int slot = 2 * w + (u0 < t0 ? 1 : 0);
        const float l = a.sk_lse[(int64_t)slot * kSkRows + r];
        if (l == -INFINITY) continue;
        const float m_new = fmaxf(M, l);
        tot = (M == -INFINITY ? 0.f : tot * expf(M - m_new)) + expf(l - m_new);
        M = m_new;
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float lse_out = -INFINITY;
    if (M != -INFINITY) {
        const float L = M + logf(tot);
        for (int w = w0; w < P; ++w) {
            const int64_t u0 = sk_start(U, w, P), u1 = sk_start(U, w + 1, P);
            if (u0 >= t1) break;
            if (u1 == u0) continue;
            const int64_t row = (int64_t)(2 * w + (u0 < t0 ? 1 : 0)) * kSkRows + r;
            const f32x4_t x = __builtin_nontemporal_load((const f32x4_t*)(a.sk_o + row * a.D + d));
            acc += expf(a.sk_lse[row] - L) * x;
        }
        lse_out = L;
    }
    store4(a.o, a.os, a.o_bf16, a.H, a.Sq, (int64_t)bh * a.Sq + s, d, acc);
    if (d == 0) a.lse[(int64_t)bh * a.Sq + s] = lse_out;
}

__global__ __launch_bounds__(kThreads) void fill_empty_kernel(void* o, Strides os, int o_bf16, float* lse, int H,
                                                              int Sq, int D, int64_t rows) {
    const int lanes_per_row = D / 4;
    const int rows_per_block = kThreads / lanes_per_row;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / lanes_per_row;
    const int d = 4 * (threadIdx.x % lanes_per_row);
    if (row >= rows) return;
    store4(o, os, o_bf16, H, Sq, row, d, f32x4_t{0.f, 0.f, 0.f, 0.f});
    if (d == 0) lse[row] = -INFINITY;
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.B * a.H * a.Sq;
    const int rows_per_block = kThreads / (a.D / 4);
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (a.n <= 2)
        hipLaunchKernelGGL(merge_kernel<2>, grid, block, 0, stream, a);
    else if (a.n <= 4)
        hipLaunchKernelGGL(merge_kernel<4>, grid, block, 0, stream, a);
    else if (a.n <= 8)
        hipLaunchKernelGGL(merge_kernel<8>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(merge_kernel<16>, grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_sk_fixup(const SkFixupArgs& a, hipStream_t stream) {
    const int n_tail = a.n_q - a.n_dp;
    if (n_tail <= 0) return hipSuccess;
    if ((a.D != 64 && a.D != 128) || a.sk_wgs <= 0 || a.T <= 0) return hipErrorInvalidValue;
    const int blocks_per_tile = kSkRows / (kThreads / (a.D / 4));
    const int64_t blocks = (int64_t)n_tail * blocks_per_tile;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(sk_fixup_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fill_empty(void* o, Strides os, int o_bf16, float* lse, int B, int H, int Sq, int D,
                             hipStream_t stream) {
    const int64_t rows = (int64_t)B * H * Sq;
    const int rows_per_block = kThreads / (D / 4);
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_empty_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, o, os, o_bf16, lse, H,
                       Sq, D, rows);
    return hipGetLastError();
}

}  // namespace lsdit
