// Chunk attention forward with fp32 inputs and fp32 arithmetic throughout.
//
// Same blockwise online-softmax evaluation as the bf16 MFMA kernel (NVIDIA
// Technical Blog "Scaling AI Inference Across Multiple GPUs Using NVIDIA
// TensorRT with Multi-Device Inference Support", section "Ring Attention"),
// on the vector ALU: this path exists for fp32 workloads that need ~1e-5
// agreement, not for throughput.
//
// A workgroup of 256 threads owns 64 query rows of one head; four
// neighbouring lanes share a row, each holding a quarter of the head
// dimension of Q and of the output accumulator.  Key/value tiles of 32 rows
// are staged in LDS; a score is four partial dot products combined with two
// lane shuffles.
#include "kernels.h"

#include <math.h>
#include <stddef.h>

namespace lsdit {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994531f;
constexpr int kRows = 64;   // query rows per workgroup
constexpr int kBK = 32;     // keys per tile
constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a, int n_qt, float c) {
    constexpr int DQ = D / 4;  // dims per lane
    __shared__ __attribute__((aligned(16))) float Ks[kBK][D + 4];
    __shared__ __attribute__((aligned(16))) float Vs[kBK][D + 4];

    const int tid = threadIdx.x;
    const int part = tid & 3;
    const int bh = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
    const int b = bh / a.H, h = bh % a.H;
    const int qrow = qt * kRows + (tid >> 2);
    const int qrow_c = qrow < a.Sq ? qrow : a.Sq - 1;
    const float* qp = (const float*)a.q + b * a.qs.b + h * a.qs.h + (int64_t)qrow_c * a.qs.s + part * DQ;
    const float* kp = (const float*)a.k + b * a.ks.b + h * a.ks.h;
    const float* vp = (const float*)a.v + b * a.vs.b + h * a.vs.h;

    float qv[DQ], o[DQ];
#pragma unroll
    for (int d = 0; d < DQ; ++d) {
        qv[d] = qp[d];
        o[d] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;

    // the chunk list, in processing order (read through the kernel-argument pointer)
    const int* const arg_rows =
        (const int*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(FwdArgs, chunk_row));
    const int* const arg_lens =
        (const int*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(FwdArgs, chunk_len));
    for (int ci = 0; ci < a.n_chunks; ++ci)
    for (int row0 = arg_rows[ci], len = arg_lens[ci], k0 = 0; k0 < len; k0 += kBK) {
        const int n = len - k0 < kBK ? len - k0 : kBK;
        __syncthreads();
        for (int idx = tid; idx < kBK * (D / 4); idx += kThreads) {
            const int r = idx / (D / 4), c4 = idx % (D / 4);
            const int key = row0 + k0 + (r < n ? r : n - 1);
            *(f32x4_t*)&Ks[r][4 * c4] = *(const f32x4_t*)(kp + (int64_t)key * a.ks.s + 4 * c4);
            *(f32x4_t*)&Vs[r][4 * c4] = *(const f32x4_t*)(vp + (int64_t)key * a.vs.s + 4 * c4);
        }
        __syncthreads();

        float s[kBK];
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < kBK; ++jj) {
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < DQ; ++d) acc = __builtin_fmaf(qv[d], Ks[jj][part * DQ + d], acc);
            acc += __shfl_xor(acc, 1, 4);
            acc += __shfl_xor(acc, 2, 4);
            s[jj] = jj < n ? acc * c : -INFINITY;
            mx = fmaxf(mx, s[jj]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int jj = 0; jj < kBK; ++jj) {
            s[jj] = exp2f(s[jj] - m_new);
            rs += s[jj];
        }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int d = 0; d < DQ; ++d) {
            float acc = o[d] * alpha;
#pragma unroll
            for (int jj = 0; jj < kBK; ++jj) acc = __builtin_fmaf(s[jj], Vs[jj][part * DQ + d], acc);
            o[d] = acc;
        }
    }

    if (qrow >= a.Sq) return;
    // normalise; fold in the running result over earlier keys if there is one (each element is
    // read, then written, by this thread: o may alias run_o)
    float lse_out = (m_run + log2f(l_run)) * kLn2, wc = 1.f / l_run, wr = 0.f;
    const float* rp = nullptr;
    if (a.run_lse) {
        const int64_t rrow = (int64_t)bh * a.Sq + qrow;
        rp = a.run_o + rrow * D + part * DQ;
        lse_out = fold_weights(lse_out, a.run_lse[rrow], wc, wr);
        wc /= l_run;
    }
    float* op = (float*)a.o + b * a.os.b + h * a.os.h + (int64_t)qrow * a.os.s + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; ++d) op[d] = rp ? o[d] * wc + wr * rp[d] : o[d] * wc;
    if (part == 0) a.lse[(int64_t)bh * a.Sq + qrow] = lse_out;
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    const int n_qt = (a.Sq + kRows - 1) / kRows;
    const int64_t n_blocks = (int64_t)a.B * a.H * n_qt;
    if (n_blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const float c = (float)((double)a.scale * 1.4426950408889634);
    hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((unsigned)n_blocks), dim3(kThreads), 0, stream, a, n_qt, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
    if (a.o_bf16) return hipErrorInvalidValue;
    if (a.D == 128) return launch_d<128>(a, stream);
    if (a.D == 64) return launch_d<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace lsdit
