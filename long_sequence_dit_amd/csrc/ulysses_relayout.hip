// Local halves of the DeepSpeed-Ulysses all-to-all (NVIDIA Technical Blog "Scaling AI
// Inference Across Multiple GPUs Using NVIDIA TensorRT with Multi-Device Inference
// Support", section "DeepSpeed Ulysses"): before attention every rank sends head group j
// of its sequence slice to rank j, and after attention the outputs travel back.
//
//   pack:   out[j][s][b][h'][d] = x[b][j*Hg + h'][s][d]     (Hg = H / n)
//   unpack: y[b][j*Hg + h'][s][d] = in[j][s][b][h'][d]
//
// The packed buffer holds each peer's part contiguously, in [S, B, Hg, D] order.  Parts
// received from ranks 0..n-1 (which hold consecutive sequence slices) therefore concatenate
// into [S_total, B, Hg, D]: head group j over the whole sequence as a strided [B, Hg, S, D]
// view (b stride Hg*D, h stride D, s stride B*Hg*D) that the attention entry points take as
// it is; the output goes back the same way.  Pure data movement, bound by HBM bandwidth:
// every lane moves 16-byte pieces, consecutive lanes cover consecutive bytes of the packed
// side, and the Hg*D elements of one (s, b) are one contiguous run on the strided side too
// when its h stride is D.
#include "kernels.h"

namespace lsdit {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
// Every byte is read once and written once: the accesses are non-temporal, so they do not
// displace other data in the caches (measured +3% pack, +6% unpack).

// Byte offset in the strided [B, H, S, D] tensor of 16-byte piece `p` of the packed tensor.
__device__ __forceinline__ int64_t strided_off(int64_t p, const RelayoutArgs& a) {
    const int64_t pieces_per_row = a.D * a.esize / 16;  // a row = the D elements of one (b, h, s)
    const int64_t dp = p % pieces_per_row;
    int64_t r = p / pieces_per_row;                        // row index in [n][S][B][Hg] order
    const int64_t hq = r % a.Hg;
    r /= a.Hg;
    const int64_t b = r % a.B;
    r /= a.B;
    const int64_t s = r % a.S;
    const int64_t j = r / a.S;
    const int64_t h = j * a.Hg + hq;
    return (b * a.st.b + h * a.st.h + s * a.st.s) * a.esize + dp * 16;
}

template <bool PACK>
__global__ __launch_bounds__(kThreads) void relayout_kernel(RelayoutArgs a) {
    const int64_t n_pieces = (int64_t)a.n * a.B * a.S * a.Hg * a.D * a.esize / 16;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t p0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; p0 < n_pieces; p0 += stride * kUnroll) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {  // all loads first, then the stores
            const int64_t p = p0 + u * stride;
            if (p < n_pieces)
                v[u] = PACK ? __builtin_nontemporal_load((const u32x4_t*)((const char*)a.src + strided_off(p, a)))
                            : __builtin_nontemporal_load((const u32x4_t*)((const char*)a.src + p * 16));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t p = p0 + u * stride;
            if (p < n_pieces) {
                if (PACK)
                    __builtin_nontemporal_store(v[u], (u32x4_t*)((char*)a.dst + p * 16));
                else
                    __builtin_nontemporal_store(v[u], (u32x4_t*)((char*)a.dst + strided_off(p, a)));
            }
        }
    }
}

}  // namespace

hipError_t launch_ulysses_relayout(const RelayoutArgs& a, bool pack, hipStream_t stream) {
    const int64_t n_pieces = (int64_t)a.n * a.B * a.S * a.Hg * a.D * a.esize / 16;
    if (n_pieces == 0) return hipSuccess;
    int64_t blocks = (n_pieces + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
    if (blocks > 8192) blocks = 8192;  // grid-stride beyond 32 workgroups per CU
    if (pack)
        hipLaunchKernelGGL(relayout_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(relayout_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lsdit
