// Chunk attention forward, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Computes, for one chunk of keys, O = softmax(scale * Q K^T) V and the
// per-row natural-log LSE, blockwise over key tiles with an online softmax
// (running max, running sum, rescale) — the evaluation that lets a rank fold
// in key/value blocks one at a time without materialising the full K and V
// (NVIDIA Technical Blog "Scaling AI Inference Across Multiple GPUs Using
// NVIDIA TensorRT with Multi-Device Inference Support", section "Ring
// Attention").  Optionally the epilogue merges the result into a running
// fp32 (O, LSE) by log-sum-exp weights.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one head):
//  * each wave owns 32 query rows; its Q rows stay in VGPRs for the whole
//    key loop as the B operand of v_mfma_f32_32x32x16_bf16;
//  * key tiles of 64 rows of K and V go HBM -> VGPR staging -> LDS, double
//    buffered, with 16-byte coalesced loads; the next tile's loads are in
//    flight while the current tile is computed;
//  * scores are computed transposed, S^T = K Q^T, so every lane holds 32
//    scores of ONE query row (lanes l and l+32 share a row); row max and row
//    sum are in-lane plus one permlane32 swap;
//  * P^T leaves the accumulator registers as bf16 and is fed directly as the
//    B operand of O^T += V^T P^T.  The MFMA k index is a relabelling of the
//    keys, so V^T is read from the row-major V tile with ds_read_b64_tr_b16
//    at the matching key rows;
//  * exponentials are base 2 with scale*log2(e) folded into one FMA.
// Workgroups are remapped so that each XCD (workgroups are dealt to the 8
// XCDs round-robin) runs consecutive query tiles of the same head, which
// then share K/V tiles in that XCD's L2.
#include "kernels.h"

#include <math.h>

namespace lsdit {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

template <int D>
struct Cfg {
    static constexpr int NW = 4;                 // waves per workgroup
    static constexpr int NT = NW * 64;           // threads per workgroup
    static constexpr int BQ = 32 * NW;           // query rows per workgroup
    static constexpr int BK = 64;                // keys per tile
    static constexpr int LDK = D + 8;            // K row pitch (elements): conflict-free 16 B row reads
    static constexpr int LDV = D + 32;           // V row pitch: conflict-free transposed 8 B reads
    static constexpr int K_ELEMS = BK * LDK;
    static constexpr int V_ELEMS = BK * LDV;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * BUF_ELEMS * 2;
    static constexpr int CHUNKS = D / 8;         // 16-byte chunks per row
    static constexpr int LOADS = BK * CHUNKS / NT;  // 16-byte loads per thread per tensor per tile
    static_assert(BK * CHUNKS % NT == 0, "tile must split evenly over the threads");
};

// Workgroups are dispatched to the 8 XCDs round-robin; give XCD x a contiguous
// range of logical tiles so its concurrently resident workgroups share K/V.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    constexpr int X = 8;
    const int q = n / X, r = n % X;
    const int xcd = bid % X, slot = bid / X;
    return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// {x of lane l%32, x of lane l%32 + 32} on every lane.
__device__ __forceinline__ void half_pair(float x, float& a, float& b) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}

template <int D>
__global__ __launch_bounds__(Cfg<D>::NT, 2) void fwd_bf16_kernel(FwdArgs a, int n_qt, float c) {
    using C = Cfg<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned short smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5;  // which half of the wave (MFMA k-half)
    const int tile = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = tile / n_qt, qt = tile % n_qt;
    const int b = bh / a.H, h = bh % a.H;

    const unsigned short* qp = (const unsigned short*)a.q + b * a.qs.b + h * a.qs.h;
    const unsigned short* kp = (const unsigned short*)a.k + b * a.ks.b + h * a.ks.h;
    const unsigned short* vp = (const unsigned short*)a.v + b * a.vs.b + h * a.vs.h;
    const int Skv = a.Skv;

    // ---- Q fragments: B operand, lane holds Q[row][16kk + 8hi .. +8]
    const int qrow = qt * C::BQ + wave * 32 + (lane & 31);
    const int qrow_c = qrow < a.Sq ? qrow : a.Sq - 1;
    bf16x8_t qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = *(const bf16x8_t*)(qp + (int64_t)qrow_c * a.qs.s + 16 * kk + 8 * hi);

    f32x16_t acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    float m_run = -INFINITY;  // running max of scale*log2(e)*s
    float l_run = 0.f;        // this lane's share of the running row sum

    const int nkt = (Skv + C::BK - 1) / C::BK;
    u32x4_t kst[C::LOADS], vst[C::LOADS];

    auto gload = [&](int t) {
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int idx = tid + i * C::NT;
            const int row = idx / C::CHUNKS, ch = idx % C::CHUNKS;
            int key = t * C::BK + row;
            key = key < Skv ? key : Skv - 1;
            kst[i] = *(const u32x4_t*)(kp + (int64_t)key * a.ks.s + ch * 8);
            vst[i] = *(const u32x4_t*)(vp + (int64_t)key * a.vs.s + ch * 8);
        }
    };
    auto swrite = [&](int buf) {
        unsigned short* Ks = smem + buf * C::BUF_ELEMS;
        unsigned short* Vs = Ks + C::K_ELEMS;
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int idx = tid + i * C::NT;
            const int row = idx / C::CHUNKS, ch = idx % C::CHUNKS;
            *(u32x4_t*)(Ks + row * C::LDK + ch * 8) = kst[i];
            *(u32x4_t*)(Vs + row * C::LDV + ch * 8) = vst[i];
        }
    };

    gload(0);
    swrite(0);
    __syncthreads();

    // transposed-read addressing for the V^T operand (see header comment)
    const int g = lane >> 4, j = lane & 15;
    const int v_row0 = 4 * (g >> 1) + (j >> 2);
    const int v_col0 = 16 * (g & 1) + 4 * (j & 3);

    for (int t = 0; t < nkt; ++t) {
        const int buf = t & 1;
        if (t + 1 < nkt) gload(t + 1);
        const unsigned short* Ks = smem + buf * C::BUF_ELEMS;
        const unsigned short* Vs = Ks + C::K_ELEMS;

        // ---- S^T = K Q^T for 2 blocks of 32 keys
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const bf16x8_t kf = *(const bf16x8_t*)(Ks + (kb * 32 + (lane & 31)) * C::LDK + 16 * kk + 8 * hi);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[kb], 0, 0, 0);
            }
        }
        // ---- mask keys past the end of the chunk (last tile only)
        const int valid = Skv - t * C::BK;
        if (valid < C::BK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (key >= valid) s[kb][r] = -INFINITY;
                }
        }
        // ---- online softmax (base 2, scaled domain)
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        float m0, m1;
        half_pair(mx, m0, m1);
        const float m_new = fmaxf(m_run, fmaxf(m0, m1) * c);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_new));
                s[kb][r] = p;
                rs += p;
            }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;

        // ---- P^T as bf16 B operands: (kb, st) covers accumulator regs 8st..8st+7 of block kb
        bf16x8_t pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                u32x4_t w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = pack_bf16(s[kb][8 * st + 2 * e], s[kb][8 * st + 2 * e + 1]);
                pf[kb * 2 + st] = __builtin_bit_cast(bf16x8_t, w);
            }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const unsigned short* base = Vs + (16 * ks + v_row0) * C::LDV + 32 * dt + v_col0;
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)base);
                const i16x4_t hi8 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + 8 * C::LDV));
                u32x4_t w;
                const u32x2_t wl = __builtin_bit_cast(u32x2_t, lo), wh = __builtin_bit_cast(u32x2_t, hi8);
                w[0] = wl[0];
                w[1] = wl[1];
                w[2] = wh[0];
                w[3] = wh[1];
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pf[ks], acc[dt],
                                                                  0, 0, 0);
            }
        }

        if (t + 1 < nkt) swrite(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: normalise, LSE, optional merge into the running result, store
    float l0, l1;
    half_pair(l_run, l0, l1);
    const float l_tot = l0 + l1;
    const float inv_l = 1.f / l_tot;
    float lse2 = m_run + log2f(l_tot);  // log2 domain
    float wa = 0.f, wb = inv_l;          // out = wa * prev + wb * acc
    const int64_t lrow = (int64_t)bh * a.Sq + qrow;
    if (a.prev_o != nullptr && qrow < a.Sq) {
        const float lp = a.prev_lse[lrow] * kLog2e;
        const float M = fmaxf(lp, lse2);
        const float ea = fast_exp2(lp - M), eb = fast_exp2(lse2 - M);
        const float tot = ea + eb;
        wa = ea / tot;
        wb = eb / tot * inv_l;
        lse2 = M + log2f(tot);
    }
    if (qrow < a.Sq) {
        const float* pp = a.prev_o ? a.prev_o + b * a.ps.b + h * a.ps.h + (int64_t)qrow * a.ps.s : nullptr;
        if (a.o_bf16) {
            unsigned short* op = (unsigned short*)a.o + b * a.os.b + h * a.os.h + (int64_t)qrow * a.os.s;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = 32 * dt + 8 * r4 + 4 * hi;
                    float x[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = acc[dt][4 * r4 + e] * wb;
                    if (pp) {
                        const f32x4_t pv = *(const f32x4_t*)(pp + d);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] += wa * pv[e];
                    }
                    u32x2_t w;
                    w[0] = pack_bf16(x[0], x[1]);
                    w[1] = pack_bf16(x[2], x[3]);
                    *(u32x2_t*)(op + d) = w;
                }
        } else {
            float* op = (float*)a.o + b * a.os.b + h * a.os.h + (int64_t)qrow * a.os.s;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = 32 * dt + 8 * r4 + 4 * hi;
                    f32x4_t x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = acc[dt][4 * r4 + e] * wb;
                    if (pp) {
                        const f32x4_t pv = *(const f32x4_t*)(pp + d);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] += wa * pv[e];
                    }
                    *(f32x4_t*)(op + d) = x;
                }
        }
    }
    // prev_lse may alias lse: the store depends on the loaded value, so it cannot overtake it.
    if (qrow < a.Sq && hi == 0) a.lse[lrow] = lse2 * kLn2;
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    using C = Cfg<D>;
    static bool attr_set[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !attr_set[dev]) {
        e = hipFuncSetAttribute((const void*)fwd_bf16_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                C::LDS_BYTES);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) attr_set[dev] = true;
    }
    const int n_qt = (a.Sq + C::BQ - 1) / C::BQ;
    const int64_t n_tiles = (int64_t)a.B * a.H * n_qt;
    if (n_tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const float c = (float)((double)a.scale * 1.4426950408889634);
    hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3((unsigned)n_tiles), dim3(C::NT), C::LDS_BYTES, stream, a, n_qt, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
    if (a.D == 128) return launch_d<128>(a, stream);
    if (a.D == 64) return launch_d<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace lsdit
