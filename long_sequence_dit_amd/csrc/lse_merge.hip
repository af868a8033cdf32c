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
// O = 0, LSE = -inf.  A NaN LSE in any part (a NaN query row, or a NaN key,
// makes its chunk's LSE NaN) makes the row's O and LSE NaN, as attention over
// all the keys in one pass gives: the running maximum below ignores NaN, so a
// flag carries it.
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
    bool nan = false;
    for (int c0 = 0; c0 < n; c0 += kBatch) {
        float l[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) l[u] = c0 + u < n ? a.lse_parts[c0 + u][row] : -INFINITY;
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            mb = fmaxf(mb, l[u]);
            nan |= l[u] != l[u];
        }
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
    if (nan) {
        acc = f32x4_t{NAN, NAN, NAN, NAN};
        lse_out = NAN;
    }
    store4(a.o, a.os, a.o_bf16, a.H, a.Sq, row, d, acc);
    // lse_parts[0] may alias lse: this store depends on every load of it above.
    if (d == 0) a.lse[row] = lse_out;
}

// The balanced tail of the forward kernels (FwdArgs) left, for each query tile j of the tail,
// fp32 partials over consecutive runs of its T key tiles.  TailRuns lists their slots.
//  * Runs of equal unit ranges (sk_parts == 0): one per run whose range meets [jT, (j+1)T).  The
//    first is the last run starting at or before jT: w = floor(((jT + 1) P - 1) / U) for P runs
//    over U units (runs may be empty when U < P).  A run that starts before jT continues into
//    tile j as its second segment (slot P + j - 1, sk_slot); the others start in tile j (slot w).
//  * r parts per tile (sk_parts == r): part p of tile j is run p * n_tail + j, in that slot.
// The runs merge by the LSE rule above; a tile's rows are read and written once.
struct TailRuns {
    int j, P, parts, n_tail, i;
    // runs of equal units: run w starts at unit b, U w = b P + rm; U = q P + ru
    int64_t t0, t1, q, ru, w, b, rm;
    __device__ TailRuns(const SkFixupArgs& a, int j_) : j(j_), P(a.sk_wgs), parts(a.sk_parts), i(0) {
        n_tail = a.n_q - a.n_dp;
        const int64_t U = (int64_t)n_tail * a.T;
        t0 = (int64_t)j * a.T;
        t1 = t0 + a.T;
        w = parts > 0 ? 0 : ((t0 + 1) * P - 1) / U;
        q = U / P;
        ru = U - q * P;
        b = U * w / P;
        rm = U * w - b * P;
    }
    // the next run's slot; -2: an empty run (skip it); -1: no more runs.  Runs of equal units
    // step from one boundary floor(U w / P) to the next without dividing.
    __device__ int next() {
        if (parts > 0) return i < parts ? (i++) * n_tail + j : -1;
        if (w >= P || b >= t1) return -1;
        int64_t b2 = b + q, rm2 = rm + ru;
        if (rm2 >= P) {
            rm2 -= P;
            b2 += 1;
        }
        const int slot = b2 == b ? -2 : sk_slot((int)w, b < t0 ? 1 : 0, j, P);
        w += 1;
        b = b2;
        rm = rm2;
        return slot;
    }
};

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
    TailRuns runs(a, j);

    // a running result over earlier keys, if given, is one more part (row bh*Sq + s of run_o)
    const int64_t orow = (int64_t)bh * a.Sq + s;
    const float l_run = a.run_lse ? a.run_lse[orow] : -INFINITY;
    float M = -INFINITY, tot = 0.f;
    bool nan = l_run != l_run;
    if (l_run != -INFINITY && !nan) {
        M = l_run;
        tot = 1.f;
    }
    // The first kH runs' partial rows and LSEs are loaded at once and held in registers (a tile
    // has r parts, or about P / n_tail + 1 runs of equal units: rarely more), with the running
    // result's row, so that one round trip to memory covers them; runs past those (a slot of -1
    // ends the list, and every later one is -1 too; -2, an empty run, is skipped) follow four
    // at a time, in two passes.  Either way the parts combine in run order.
    constexpr int kH = 8, kB = 4;
    int sh[kH];
    bool end = false;
#pragma unroll
    for (int u = 0; u < kH; ++u) {
        sh[u] = end ? -1 : runs.next();
        end |= sh[u] == -1;
    }
    const bool more = !end;
    const TailRuns rest = runs;  // positioned after the held runs
    f32x4_t xh[kH];
    float lh[kH];
    const f32x4_t x_run = l_run != -INFINITY && !nan ? *(const f32x4_t*)(a.run_o + orow * a.D + d)
                                                     : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kH; ++u) {
        const int64_t row = (int64_t)(sh[u] >= 0 ? sh[u] : 0) * kSkRows + r;
        xh[u] = sh[u] >= 0 ? __builtin_nontemporal_load((const f32x4_t*)(a.sk_o + row * a.D + d))
                           : f32x4_t{0.f, 0.f, 0.f, 0.f};
        lh[u] = sh[u] >= 0 ? a.sk_lse[row] : -INFINITY;
    }
    auto fold = [&](float l) {
        nan |= l != l;
        if (l == -INFINITY || l != l) return;
        const float m_new = fmaxf(M, l);
        tot = (M == -INFINITY ? 0.f : tot * expf(M - m_new)) + expf(l - m_new);
        M = m_new;
    };
#pragma unroll
    for (int u = 0; u < kH; ++u) fold(lh[u]);
    if (more) {
        TailRuns it = rest;
        for (;;) {
            int sl[kB];
            float lb[kB];
            bool e = false;
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                sl[u] = e ? -1 : it.next();
                e |= sl[u] == -1;
            }
#pragma unroll
            for (int u = 0; u < kB; ++u) lb[u] = sl[u] >= 0 ? a.sk_lse[(int64_t)sl[u] * kSkRows + r] : -INFINITY;
#pragma unroll
            for (int u = 0; u < kB; ++u) fold(lb[u]);
            if (e) break;
        }
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float lse_out = -INFINITY;
    if (M != -INFINITY) {
        const float L = M + logf(tot);
        if (l_run != -INFINITY) acc = expf(l_run - L) * x_run;
#pragma unroll
        for (int u = 0; u < kH; ++u)
            if (sh[u] >= 0) acc += expf(lh[u] - L) * xh[u];
        if (more) {
            TailRuns it = rest;
            for (;;) {
                int sl[kB];
                f32x4_t x[kB];
                float wl[kB];
                bool e = false;
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    sl[u] = e ? -1 : it.next();
                    e |= sl[u] == -1;
                }
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    const int64_t row = (int64_t)(sl[u] >= 0 ? sl[u] : 0) * kSkRows + r;
                    x[u] = sl[u] >= 0 ? __builtin_nontemporal_load((const f32x4_t*)(a.sk_o + row * a.D + d))
                                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
                    wl[u] = sl[u] >= 0 ? a.sk_lse[row] : -INFINITY;
                }
#pragma unroll
                for (int u = 0; u < kB; ++u)
                    if (sl[u] >= 0) acc += expf(wl[u] - L) * x[u];
                if (e) break;
            }
        }
        lse_out = L;
    }
    if (nan) {
        acc = f32x4_t{NAN, NAN, NAN, NAN};
        lse_out = NAN;
    }
    // o and lse may alias run_o and run_lse: these stores depend on every load of them above
    store4(a.o, a.os, a.o_bf16, a.H, a.Sq, orow, d, acc);
    if (d == 0) a.lse[orow] = lse_out;
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

__global__ void wq_clear_kernel(unsigned* wq) {
    if (threadIdx.x < kWorkQueueWords / kWorkQueueStride) wq[threadIdx.x * kWorkQueueStride] = 0u;
}

hipError_t launch_wq_clear(unsigned* wq, hipStream_t stream) {
    if (!wq) return hipErrorInvalidValue;
    hipLaunchKernelGGL(wq_clear_kernel, dim3(1), dim3(64), 0, stream, wq);
    return hipGetLastError();
}

hipError_t launch_sk_fixup(const SkFixupArgs& a, hipStream_t stream) {
    const int n_tail = a.n_q - a.n_dp;
    if (n_tail <= 0) return hipSuccess;
    if ((a.D != 64 && a.D != 128) || a.sk_wgs <= 0 || a.T <= 0) return hipErrorInvalidValue;
    if (a.sk_parts < 0 || (a.sk_parts > 0 && (a.sk_parts > a.T || (int64_t)a.sk_parts * n_tail != a.sk_wgs)))
        return hipErrorInvalidValue;
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
