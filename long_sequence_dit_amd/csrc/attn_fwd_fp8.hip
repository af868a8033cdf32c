// Chunk attention forward, FP8 (OCP E4M3) inputs, fp32 accumulation, gfx950 MFMA (D = 128).
//
// The computation of the bf16 kernel — O = softmax(scale * Q K^T) V for one chunk of keys and
// the per-row natural-log LSE, blockwise over key tiles with an online softmax (NVIDIA
// Technical Blog "Scaling AI Inference Across Multiple GPUs Using NVIDIA TensorRT with
// Multi-Device Inference Support", section "Ring Attention") — on E4M3 tensors, the 8-bit
// float format that suits attention layers ("TensorRT Multi-Device Inference: Engineering
// Practices for Breaking Through Single-GPU Memory Bottlenecks", section "Why a Single GPU Is
// No Longer Enough").  Each tensor holds E4M3 codes; its values are the codes times a
// per-tensor descale.
//
// Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales): 64-deep
// contractions at twice the bf16 MFMA rate, with half the bytes per operand.
//  * S^T = K Q^T as in the bf16 kernel: 8 waves x 32 query rows, Q (B operand, 2 x 32 bytes
//    per lane) in VGPRs, K tiles of 64 keys (8 KiB) from LDS, each lane ends with 32 scores of
//    one query row.  The MFMA contracts A and B over the same (lane half, byte) positions, so
//    any assignment of d to those positions works if Q and K use the same one: lane half h
//    takes bytes 32h..32h+31 of each 64-wide d step.
//  * P^T (E4M3) is the B operand of O^T += V^T P^T.  A lane's 32 probabilities, in register
//    order, are its B bytes, which fixes which key each (lane half, byte) position stands for;
//    V^T must present the same keys in the same positions.  A pre-pass (fp8_pack_v) writes V
//    as such V^T tiles (128 rows of d x 64 key bytes, already in the LDS layout), so every
//    operand read is a plain 16-byte LDS read and every tile load is one contiguous 8 KiB.
//  * The row sum is one more MFMA per tile, v_mfma_scale_f32_16x16x128_f8f6f4 (a quarter of
//    the flops of the 32x32x64 form, half its cycles): a lane's P^T bytes are also a valid B
//    operand there (column l % 16, k group l / 16: queries 0-15 and 16-31 of both key halves),
//    and an A operand of E4M3 ones where the k group's parity equals bit 3 of the row sums both
//    halves of query n into rows 0-7 of column n and those of query n + 16 into rows 8-15.  So
//    the sum of the E4M3 probabilities (the values P.V uses) of query l % 32 lands in lane l
//    for lanes 0-15 and 48-63, and in lane l + 16 (l - 16) for lanes 16-31 (32-47).
//  * Probabilities are stored as E4M3(2^5 p): with the lazy rescale threshold 2^3, 2^5 p stays
//    <= 256 (E4M3 tops out at 448), and probabilities down to 2^-11 of the reference are
//    normal numbers; the 2^5 cancels in O = sum(P V) / sum(P) and is taken out of the LSE.
//  * Descales fold into the kernel's constants: scale * log2(e) * q_descale * k_descale
//    multiplies the scores, v_descale / l the output.
// Loads, LDS swizzles, the tile ring and the loop barrier follow the bf16 kernel.
#include "kernels.h"

#include <atomic>
#include <math.h>
#include <stddef.h>

#include <type_traits>

namespace lsdit {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
// Kernel arguments seen through the constant address space (scalar loads).
template <class T>
using kernarg_t = __attribute__((address_space(4))) const T;

constexpr int D = 128;
constexpr int NW = 8;               // waves per workgroup
constexpr int NT = NW * 64;
constexpr int BQ = 32 * NW;         // query rows per workgroup
constexpr int BK = 64;              // keys per tile
constexpr int K_ROW = D;            // bytes per K row
constexpr int TILE = kFp8TileBytes; // bytes of a K tile and of a V^T tile
constexpr int NSTAGE = 4;           // LDS buffers per tensor (the key loop is unrolled by NSTAGE)
constexpr int ITEM_ADDR = 2 * NSTAGE * TILE;  // a persistent workgroup's next item, broadcast to the waves
constexpr int LDS_BYTES = ITEM_ADDR + 16;
constexpr int BLKS = TILE / 1024;   // wave-wide 1 KiB loads per tile
constexpr int LOADERS = NW / 2;     // waves 0-3 issue the tile loads (as in the bf16 kernel)
constexpr int BLKS_PER_WAVE = BLKS / LOADERS;
static_assert(BLKS % LOADERS == 0, "tile must split evenly over the loading waves");
constexpr float kRescale = 3.0f;    // lazy-rescale threshold, log2 units
constexpr float kPShift = 5.0f;     // probabilities are stored as E4M3(2^kPShift * p)
constexpr unsigned kOnes = 0x38383838u;  // four E4M3 ones
constexpr int kUnitScale = 127;     // E8M0 block scale 2^0
constexpr float kLn2 = 0.69314718055994531f;

// Stream slots: P.V for d blocks 0..3, the row sum, then scores (kk, kb) with kb fastest.
constexpr int N_PV = 5;
constexpr int N_S = 4;
constexpr int N_SLOTS = N_PV + N_S;
constexpr int kPrefetch = 2;        // operands read this many slots ahead

__device__ __forceinline__ f32x16_t mfma(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kUnitScale, 0, kUnitScale);
}

// Row-sum MFMA (see the header): lane l's A bytes are ones where ((l >> 4) & 1) == bit 3 of l.
__device__ __forceinline__ f32x4_t mfma_rowsum(const i32x8_t& a, const i32x8_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, kUnitScale, 0, kUnitScale);
}
// The lane whose row sum belongs to the query of lane l (and the reverse).
__device__ __forceinline__ int rowsum_partner(int lane) {
    return lane < 16 || lane >= 48 ? lane : (lane < 32 ? lane + 16 : lane - 16);
}
__device__ __forceinline__ float from_lane(int src, float x) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(x)));
}

__device__ __forceinline__ int xcd_remap(int bid, int n) {
    constexpr int X = 8;
    const int q = n / X, r = n % X;
    const int xcd = bid % X, slot = bid / X;
    return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// 2^x for x <= 0, clamped to [0, 1] by the exponential instruction itself (the clamp folds into
// v_exp_f32), which also maps NaN to 0: a NaN query row (every score NaN) then adds nothing to
// the row-sum MFMA, whose zero entries would otherwise carry the NaN into the sum of the query
// that shares its MFMA column.  The NaN still reaches the row's own output through its
// reference (see the lazy rescale).
__device__ __forceinline__ float weight_exp2(float x) {
    return __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x), 0.f, 1.f);
}
// E4M3 codes of 2^8 a and 2^8 b into the low (HI false) or high 16 bits of `word`, keeping the
// other half: the scaled conversion divides by its scale operand, 2^-8 (exact).  Written as
// assembly because the compiler's form of this conversion does not keep the other half of the
// destination (it dropped the low half's conversion, measured wrong on the GPU); the result is
// read many instructions later (the next tile's P.V), so no wait state is needed after it.
template <bool HI>
__device__ __forceinline__ void pack_e4m3_x256(int& word, float a, float b) {
    const float inv = 1.f / 256.f;
    if constexpr (HI)
        asm volatile("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(word) : "v"(a), "v"(b), "s"(inv));
    else
        asm volatile("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %3" : "+v"(word) : "v"(a), "v"(b), "s"(inv));
}

__device__ __forceinline__ void half_pair(float x, float& a, float& b) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}

// IEEE maximum (NaN-propagating): one v_maximum3_f32 per call, on raw MFMA results too.  (The
// NaN-ignoring fmaxf needs its inputs quieted first, one more instruction per input that is not
// already the result of a max.)  Row maxima of scores are the only use; a NaN score makes its
// row NaN either way.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3(float a, float b, float c) { return vmax(vmax(a, b), c); }

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}

struct Rsrc {
    i32x4_t w;
};
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int num_records) {
    const unsigned long long a = (unsigned long long)base;
    Rsrc r;
    r.w[0] = (int)(unsigned)a;
    r.w[1] = (int)((unsigned)(a >> 32) & 0xFFFFu);
    r.w[2] = num_records;
    r.w[3] = 0x00020000;
    return r;
}
// Resource of one tile: the bytes [off, end) of a head's data, rebased to off (empty when off >=
// end).  The raw-buffer range check applies to the per-lane offset, not to a scalar offset, so
// each tile gets a resource of its own and rows past the data read as zeros.
__device__ __forceinline__ Rsrc tile_rsrc(const void* base, int off, int end) {
    return make_rsrc((const unsigned char*)base + off, off < end ? end - off : 0);
}

// Wave-wide 16-byte-per-lane loads into consecutive 1 KiB LDS blocks (see the bf16 kernel for
// why these are assembly: the kernel orders the LDS writes itself, by a vmcnt wait and the
// loop barrier).
template <int NB>
__device__ __forceinline__ void lds_dma(const Rsrc& rs, unsigned dst, const int (&goff)[NB]) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
        asm volatile(
            "s_nop 0\n\t"
            "buffer_load_dwordx4 %0, %1, 0 offen lds"
            :
            : "v"(goff[i]), "s"(rs.w), "{m0}"(dst + i * 1024u)
            : "memory");
}

// K tile rows (128 bytes, 8 chunks) in LDS: 16-byte chunk c of row r sits at position
// c ^ k_swz(r).  An operand read has lanes on 32 consecutive rows at one logical chunk; with
// c ^ (r & 7) alone, rows r and r + 8 land on the same banks (4 conflict cycles per read,
// measured with SQ_LDS_BANK_CONFLICT); folding bits 3-4 of the row in separates them (0
// measured).  Independent of row bit 5 (the key block), so key blocks stay 4 KiB apart.
__device__ __forceinline__ int k_swz(int row) { return (row & 7) ^ ((row >> 3) & 3); }
// V^T tile rows (64 bytes, one per d): chunk c of row d at position c ^ ((d >> 2) & 3)
// (0 conflict cycles measured).
__device__ __forceinline__ int vt_swz(int d) { return (d >> 2) & 3; }

// Key held at byte position (lane half h, byte b) of a P^T / V^T operand: byte b of a lane's
// probabilities is score f = b of that lane, i.e. accumulator element e = b & 15 of key block
// kb = b >> 4, which is key 32 kb + 8 (e >> 2) + 4 h + (e & 3).
__host__ __device__ constexpr int vt_key(int h, int b) {
    return 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * h + (b & 3);
}

// ---- V^T pre-pass: one workgroup per (b, h, key tile).  Reads 64 rows of V (zeros past Skv)
// and writes the 8 KiB V^T tile in the LDS layout the forward kernel loads verbatim:
// row d (64 bytes) holds at byte 32h + b the value of key vt_key(h, b), chunk-swizzled.
constexpr int PACK_T = 256;

__global__ __launch_bounds__(PACK_T) void fp8_pack_v_kernel(Fp8Args a, int n_kt) {
    __shared__ __attribute__((aligned(16))) unsigned char tile[BK * D];
    const int g = blockIdx.x % n_kt, bh = blockIdx.x / n_kt;
    const int b = bh / a.H, h = bh % a.H;
    const unsigned char* vp = (const unsigned char*)a.v + b * a.vs.b + h * a.vs.h;
    for (int i = threadIdx.x; i < BK * D / 16; i += PACK_T) {
        const int r = i / (D / 16), c = i % (D / 16);
        const int key = g * BK + r;
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (key < a.Skv) x = *(const u32x4_t*)(vp + (int64_t)key * a.vs.s + 16 * c);
        *(u32x4_t*)(tile + r * D + 16 * c) = x;
    }
    __syncthreads();
    unsigned char* out = (unsigned char*)a.vt + ((int64_t)bh * n_kt + g) * TILE;
    for (int i = threadIdx.x; i < TILE / 16; i += PACK_T) {
        const int d = i / 4, pos = i % 4;
        const int c = pos ^ vt_swz(d);  // logical chunk stored at this position
        const int hh = c >> 1, b0 = 16 * (c & 1);
        unsigned w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            unsigned x = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) x |= (unsigned)tile[vt_key(hh, b0 + 4 * j + u) * D + d] << (8 * u);
            w[j] = x;
        }
        *(u32x4_t*)(out + 16 * i) = u32x4_t{w[0], w[1], w[2], w[3]};
    }
}

// ---- forward kernel

struct Wave {
    f32x16_t acc[D / 32];  // O^T accumulators
    f32x4_t lacc;          // row sums (every element; lanes 16-47 hold their partner's query)
    i32x8_t qf[D / 64];    // Q bytes, B operands of the score MFMAs
    i32x8_t rs_a;          // A operand of the row-sum MFMA
    float m_run;           // reference max (scaled, log2 domain)
    float c;               // scale * log2(e) * q_descale * k_descale
};

struct Soft {
    float mt[11];
    float m_new, alpha, nb;  // nb = kPShift - 8 - m_new
    float x[16][2];
    float e[16][2];
};

__device__ __forceinline__ float sel_f(const f32x16_t (&s)[2], int f) { return s[f >> 4][f & 15]; }

__device__ __forceinline__ void pin(float& a, float& b) { asm volatile("" : "+v"(a), "+v"(b)); }

// Softmax schedule over the 9 slots of a stream: the max tree in slots 0-1 (the first key half,
// whose last score MFMA ran a slot before the second half's, in slot 0), the reference update in
// slot 2, then pair J of scores (2J, 2J+1) as a three-stage pipeline (FMA at a(J), exp at
// a(J)+1, E4M3 pack at a(J)+2) with a(J) in 3..6: at most 8 exponentials per slot.
__host__ __device__ constexpr int pair_slot(int j) { return 3 + j / 4; }

template <int POS, int J = 0>
__device__ __forceinline__ void pair_stages(float c, Soft& sm, const f32x16_t (&s)[2], i32x8_t& p) {
    if constexpr (J < 16) {
        constexpr int a = pair_slot(J);
        if constexpr (POS == a) {
            const float x0 = s[J >> 3][2 * (J & 7)], x1 = s[J >> 3][2 * (J & 7) + 1];
            sm.x[J][0] = __builtin_fmaf(x0, c, sm.nb);
            sm.x[J][1] = __builtin_fmaf(x1, c, sm.nb);
            pin(sm.x[J][0], sm.x[J][1]);
        } else if constexpr (POS == a + 1) {
            sm.e[J][0] = weight_exp2(sm.x[J][0]);
            sm.e[J][1] = weight_exp2(sm.x[J][1]);
            pin(sm.e[J][0], sm.e[J][1]);
        } else if constexpr (POS == a + 2) {
            // bytes 2J, 2J+1 of the operand: half (J & 1) of dword J / 2, E4M3 of 2^8 times the
            // weights (the scaled conversion divides by its scale operand, 2^-8: exact).  The
            // conversion keeps the other half of the dword it is given; for the low half that is a
            // stale value the high half's conversion then replaces (no zeroing needed)
            int word = p[J >> 1];
            pack_e4m3_x256<(J & 1) != 0>(word, sm.e[J][0], sm.e[J][1]);
            p[J >> 1] = word;
        }
        pair_stages<POS, J + 1>(c, sm, s, p);
    }
}

template <int POS>
__device__ __forceinline__ void softmax_slot(Wave& w, Soft& sm, const f32x16_t (&s)[2], i32x8_t& p) {
    if constexpr (POS == 0) {
        // scores 0-14 (the first key half, whose last MFMA ran a slot earlier than the second's)
#pragma unroll
        for (int i = 0; i < 5; ++i) sm.mt[i] = max3(sel_f(s, 3 * i), sel_f(s, 3 * i + 1), sel_f(s, 3 * i + 2));
    } else if constexpr (POS == 1) {
#pragma unroll
        for (int i = 5; i < 10; ++i) sm.mt[i] = max3(sel_f(s, 3 * i + 1), sel_f(s, 3 * i + 2), sel_f(s, 3 * i + 3));
        sm.mt[10] = max3(sel_f(s, 15), sel_f(s, 31), sm.mt[0]);
        sm.mt[1] = max3(sm.mt[1], sm.mt[2], sm.mt[3]);
    } else if constexpr (POS == 2) {
        const float mx = max3(max3(sm.mt[1], sm.mt[4], sm.mt[5]), max3(sm.mt[6], sm.mt[7], sm.mt[8]),
                              vmax(sm.mt[9], sm.mt[10]));
        float m0, m1;
        half_pair(mx, m0, m1);
        // lazy rescale: the reference moves only when the row max exceeds it by > kRescale (or
        // is NaN: then the reference, the rescale factor and so the row's output become NaN), so
        // p <= 2^kRescale and 2^kPShift p fits E4M3; lanes l and l+32 agree.  The exponentials
        // give 2^(kPShift - 8) p <= 1 (see weight_exp2), and the E4M3 conversion scales by 2^8
        const float m_tile = vmax(m0, m1) * w.c;
        sm.m_new = !(m_tile <= w.m_run + kRescale) ? m_tile : w.m_run;
        sm.alpha = fast_exp2(w.m_run - sm.m_new);
        w.m_run = sm.m_new;
        sm.nb = (kPShift - 8.f) - sm.m_new;
    }
    pair_stages<POS>(w.c, sm, s, p);
}

template <int POS = 0>
__device__ __forceinline__ void softmax_all(Wave& w, Soft& sm, const f32x16_t (&s)[2], i32x8_t& p) {
    if constexpr (POS < N_SLOTS) {
        softmax_slot<POS>(w, sm, s, p);
        softmax_all<POS + 1>(w, sm, s, p);
    }
}

// Per-lane LDS read offsets (bytes, buffer 0): V^T operand of d block dt at va[j] + 2048 dt,
// K operand of (kk, kb) at ka[kk][j] + 4096 kb; j picks the operand's two 16-byte halves.
struct Addr {
    unsigned va[2];
    unsigned ka[2][2];
};

// The 32-byte operand of slot SLOT (V^T / K); vb / kb_ carry the buffer offsets.
template <int SLOT>
__device__ __forceinline__ i32x8_t read_opnd(const Addr& ad, unsigned vb, unsigned kb_) {
    u32x4_t lo, hi;
    if constexpr (SLOT < 4) {
        lo = *(const lds_u32x4_t*)(size_t)(ad.va[0] + vb + 2048u * SLOT);
        hi = *(const lds_u32x4_t*)(size_t)(ad.va[1] + vb + 2048u * SLOT);
    } else {
        constexpr int sl = SLOT - N_PV, kk = sl >> 1, kb = sl & 1;
        lo = *(const lds_u32x4_t*)(size_t)(ad.ka[kk][0] + kb_ + 4096u * kb);
        hi = *(const lds_u32x4_t*)(size_t)(ad.ka[kk][1] + kb_ + 4096u * kb);
    }
    return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Slots that read an operand: every slot but the row sum.
__host__ __device__ constexpr bool reads(int slot) { return slot != 4; }
// Index of slot's operand in the read sequence (the row-sum slot reads nothing).
__host__ __device__ constexpr int read_idx(int slot) { return slot < 4 ? slot : slot - 1; }

template <bool DO_PV, bool DO_S, bool DO_SM, int SLOT>
__device__ __forceinline__ void stream_slots(Wave& w, const Addr& ad, unsigned vb, unsigned kb_,
                                             i32x8_t (&ring)[kPrefetch], const i32x8_t& p_prev,
                                             const f32x16_t (&s_cur)[2], f32x16_t (&s)[2], i32x8_t& p_cur,
                                             Soft& sm) {
    constexpr int last = DO_S ? N_SLOTS : N_PV;
    if constexpr (SLOT < last) {
        if constexpr (SLOT < 4) {
            w.acc[SLOT] = mfma(ring[read_idx(SLOT) % kPrefetch], p_prev, w.acc[SLOT]);
        } else if constexpr (SLOT == 4) {
            w.lacc = mfma_rowsum(w.rs_a, p_prev, w.lacc);
        } else {
            constexpr int sl = SLOT - N_PV, kk = sl >> 1, kb = sl & 1;
            if constexpr (kk == 0) {
                const f32x16_t zero = {};
                s[kb] = mfma(ring[read_idx(SLOT) % kPrefetch], w.qf[kk], zero);
            } else {
                s[kb] = mfma(ring[read_idx(SLOT) % kPrefetch], w.qf[kk], s[kb]);
            }
        }
        // read the operand kPrefetch reads ahead (the slot that consumes it)
        if constexpr (reads(SLOT)) {
            constexpr int nxt = read_idx(SLOT) + kPrefetch;                 // read index
            constexpr int nslot = nxt < 4 ? nxt : nxt + 1;                  // its slot
            if constexpr (nslot < last) ring[nxt % kPrefetch] = read_opnd<nslot>(ad, vb, kb_);
        }
        if constexpr (DO_SM) softmax_slot<SLOT>(w, sm, s_cur, p_cur);
        __builtin_amdgcn_sched_barrier(0);
        stream_slots<DO_PV, DO_S, DO_SM, SLOT + 1>(w, ad, vb, kb_, ring, p_prev, s_cur, s, p_cur, sm);
    }
}

// One stream: P.V (and row sum) of the tile at v0 with probabilities p_prev (if DO_PV), the
// softmax of s_cur into p_cur (if DO_SM), the scores of the tile at k0 into s (if DO_S).
template <bool DO_PV, bool DO_S, bool DO_SM>
__device__ __forceinline__ void stream(Wave& w, const Addr& ad, unsigned v0, unsigned k0, const i32x8_t& p_prev,
                                       const f32x16_t (&s_cur)[2], f32x16_t (&s)[2], i32x8_t& p_cur, Soft& sm) {
    static_assert(!DO_SM || (DO_PV && DO_S), "the softmax runs over a full stream");
    constexpr int first = DO_PV ? 0 : N_PV;
    static_assert(kPrefetch == 2, "the stream's first reads below assume two in flight");
    i32x8_t ring[kPrefetch];
    // the stream's first kPrefetch reads
    if constexpr (first == 0) {
        ring[0] = read_opnd<0>(ad, v0, k0);
        ring[1] = read_opnd<1>(ad, v0, k0);
    } else {
        // score-only stream: reads are indexed from the first score slot
        ring[read_idx(N_PV) % kPrefetch] = read_opnd<N_PV>(ad, v0, k0);
        ring[read_idx(N_PV + 1) % kPrefetch] = read_opnd<N_PV + 1>(ad, v0, k0);
    }
    __builtin_amdgcn_sched_barrier(0);
    stream_slots<DO_PV, DO_S, DO_SM, first>(w, ad, v0, k0, ring, p_prev, s_cur, s, p_cur, sm);
}

__global__ __launch_bounds__(NT, 1) void fwd_fp8_kernel(Fp8Args a, int n_qt, int n_kt) {
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];  // no static LDS: starts at address 0
    static_assert(BQ == kSkRows, "stream-K slots hold one query tile");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_q = a.B * a.H * n_qt;

    // This workgroup's items (see Fp8Args, FwdArgs), each one or two segments (query tile, run of
    // key tiles): a whole query tile, or a run of the balanced tail's (query tile, key tile)
    // units, which spans at most two query tiles.  The first item is the workgroup's own index; a
    // persistent workgroup then takes items from the work queues (wq_next) until they are
    // empty.  As in the bf16 kernel, each iteration re-derives its segment, the arguments
    // (through an opaque pointer) and the lane index, so nothing computed from them is held
    // across the key loop, and the segment bounds are made wave-uniform.
    int seg = 0, bid = 0;
    unsigned wq_empty = 0;  // queues found empty (thread 0's)
    for (int it = 0;; ++it) {
        const kernarg_t<Fp8Args>* ap = (const kernarg_t<Fp8Args>*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        const kernarg_t<Fp8Args>& ar = *ap;
        const int n_whole = ar.sk_wgs == 0 ? n_q : ar.n_dp;
        if (seg == 0) {
            if (it == 0) {
                bid = wg_logical((int)blockIdx.x, (int)gridDim.x, ar.wg_order);
            } else {
                if (ar.persist == 0) break;
                // thread 0 takes the next item as soon as its wave is done (the atomic's latency
                // overlaps the drain of the last item's stores) and broadcasts it through an LDS
                // word: every wave read the word's last value before the barrier that ends the
                // last segment's prologue, which thread 0 has passed since
                int* const item = (int*)(smem + ITEM_ADDR);
                if (tid == 0) {
                    const int xcd = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11));  // XCC_ID[3:0]
                    *item = wq_next(ar.wq, xcd, (int)gridDim.x, n_whole, n_whole + ar.sk_wgs, wq_empty);
                }
                // every wave is done with the last item's tiles (and no load is in flight) before
                // the next item's prologue rewrites LDS
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                __syncthreads();
                bid = __builtin_amdgcn_readfirstlane(*(volatile int*)item);
                if (bid < 0) break;
            }
        }
        int lane = tid & 63;
        asm volatile("" : "+v"(lane));
        const int hi = lane >> 5;
        int sk_slot_ = -1, gidx, g_first, nkt;
        if (bid < n_whole) {
            if (seg > 0) {
                seg = 0;
                continue;
            }
            gidx = xcd_remap(bid, n_whole);
            g_first = 0;
            nkt = n_kt;
        } else {
            // the tail's runs in plain order: the XCDs take them round-robin (or from their
            // queues by b % 8), so the runs on one XCD are 8 apart.  Runs of equal unit ranges
            // start 8 U / P units apart, often a whole number of query tiles (the ring share) or
            // half of one (the full sequence): they stream the same key tiles together and
            // share them in the L2 (remapped to consecutive runs, their starts spread over the
            // whole key range).  Parts are numbered part-major, so an XCD's runs at one time are
            // mostly the same part, the same key range, of different tail tiles.
            const int sk_w = bid - ar.n_dp;
            if (ar.sk_parts > 0) {
                // part p = sk_w / n_tail of tail tile sk_w % n_tail: one segment
                if (seg > 0) {
                    seg = 0;
                    continue;
                }
                const int n_tail = n_q - ar.n_dp, p = sk_w / n_tail;
                gidx = ar.n_dp + sk_w % n_tail;
                g_first = (int)((int64_t)n_kt * p / ar.sk_parts);
                nkt = (int)((int64_t)n_kt * (p + 1) / ar.sk_parts) - g_first;
                sk_slot_ = sk_w;
            } else {
                const int64_t U = (int64_t)(n_q - ar.n_dp) * n_kt;
                const int64_t u0 = sk_start(U, sk_w, ar.sk_wgs), u1 = sk_start(U, sk_w + 1, ar.sk_wgs);
                const int64_t cut = (u0 / n_kt + 1) * n_kt;
                const int64_t s0 = seg == 0 ? u0 : cut, s1 = seg == 0 ? (u1 < cut ? u1 : cut) : u1;
                if (seg > 1 || s0 >= s1) {
                    seg = 0;
                    continue;
                }
                sk_slot_ = sk_slot(sk_w, seg, (int)(s0 / n_kt), ar.sk_wgs);
                gidx = ar.n_dp + (int)(s0 / n_kt);
                g_first = (int)(s0 % n_kt);
                nkt = (int)(s1 - s0);
            }
        }
        gidx = __builtin_amdgcn_readfirstlane(gidx);
        g_first = __builtin_amdgcn_readfirstlane(g_first);
        nkt = __builtin_amdgcn_readfirstlane(nkt);
        sk_slot_ = __builtin_amdgcn_readfirstlane(sk_slot_);
        if (seg > 0) {
            // every wave is done with the previous segment's tiles (and no load is in flight)
            // before this segment's prologue rewrites LDS
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __syncthreads();
        }
        ++seg;
        const int bh = gidx / n_qt, qt = gidx % n_qt;
        const int b = bh / ar.H, h = bh % ar.H;
        const unsigned char* qp = (const unsigned char*)ar.q + b * ar.qs.b + h * ar.qs.h;
        const unsigned char* kp = (const unsigned char*)ar.k + b * ar.ks.b + h * ar.ks.h;
        const int Skv = ar.Skv;

        Wave w;
        w.c = ar.c;
        w.m_run = -INFINITY;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) w.acc[dt][r] = 0.f;
        w.lacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        {
            const int ra = ((lane >> 4) & 1) == ((lane & 15) >> 3) ? (int)kOnes : 0;
#pragma unroll
            for (int r = 0; r < 8; ++r) w.rs_a[r] = ra;
        }
        asm volatile("" : "+v"(w.rs_a));  // kept in registers, not rebuilt before every use

        // Q bytes: lane (row, half h) holds d = 64 kk + 32 h .. +32 of its row
        const int qrow = qt * BQ + wave * 32 + (lane & 31);
        const int qrow_c = qrow < ar.Sq ? qrow : ar.Sq - 1;
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) {
            const u32x4_t* src = (const u32x4_t*)(qp + (int64_t)qrow_c * ar.qs.s + 64 * kk + 32 * hi);
            const u32x4_t lo = src[0], hi4 = src[1];
            w.qf[kk] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                               (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
        }

        // tile loads: K rows through a per-lane swizzled offset, V^T tiles verbatim
        const int k_rs = (int)ar.ks.s;  // bytes per K row step
        const int k_end = (Skv - 1) * k_rs + D;  // bytes of a head's K rows
        const unsigned char* const vtp = (const unsigned char*)ar.vt + (int64_t)bh * n_kt * TILE;
        int k_goff[BLKS_PER_WAVE], v_goff[BLKS_PER_WAVE];
#pragma unroll
        for (int i = 0; i < BLKS_PER_WAVE; ++i) {
            const int blk = wave * BLKS_PER_WAVE + i;
            const int row = blk * 8 + lane / 8, slot = lane % 8;
            k_goff[i] = row * k_rs + (slot ^ k_swz(row)) * 16;
            v_goff[i] = blk * 1024 + lane * 16;
        }
        // LDS byte offsets of the tile buffers: tile g of the segment (key tile g_first + g) sits in
        // buffer g mod NSTAGE
        auto kbuf = [&](int t) { return (unsigned)((t % NSTAGE) * TILE); };
        auto vbuf = [&](int t) { return (unsigned)((NSTAGE + t % NSTAGE) * TILE); };
        auto load_k = [&](int g) {
            if (wave < LOADERS)
                lds_dma<BLKS_PER_WAVE>(tile_rsrc(kp, (g_first + g) * BK * k_rs, k_end),
                                       kbuf(g) + wave * BLKS_PER_WAVE * 1024, k_goff);
        };
        auto load_v = [&](int g) {
            if (wave < LOADERS)
                lds_dma<BLKS_PER_WAVE>(tile_rsrc(vtp, (g_first + g) * TILE, n_kt * TILE),
                                       vbuf(g) + wave * BLKS_PER_WAVE * 1024, v_goff);
        };

        // per-lane operand offsets
        Addr ad;
        {
            const int l32 = lane & 31;
            ad.va[0] = l32 * 64 + (((2 * hi) ^ vt_swz(l32)) * 16);
            ad.va[1] = l32 * 64 + (((2 * hi + 1) ^ vt_swz(l32)) * 16);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int j = 0; j < 2; ++j) ad.ka[kk][j] = l32 * K_ROW + (((4 * kk + 2 * hi + j) ^ k_swz(l32)) * 16);
            // opaque to the compiler, so that buffer and block offsets stay additions it folds into
            // the reads' offset fields (with the offsets' bits known disjoint it may turn them
            // into ORs computed per read)
            asm volatile("" : "+v"(ad.va[0]), "+v"(ad.va[1]), "+v"(ad.ka[0][0]), "+v"(ad.ka[0][1]), "+v"(ad.ka[1][0]),
                         "+v"(ad.ka[1][1]));
        }

        // scores of keys at or past `valid` in a tile -> -inf (key of element (kb, r) is
        // 32 kb + 8 (r >> 2) + 4 hi + (r & 3))
        auto mask = [&](f32x16_t(&s)[2], int valid) {
            if (valid < BK) {
                const int lim = valid - 4 * hi;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = -INFINITY;
            }
        };
        auto valid_of = [&](int t) { return Skv - (g_first + t) * BK; };

        // prologue (as in the bf16 kernel, LDS needs no clearing: every buffer is loaded whole
        // before it is read; rows past the end read as zeros and are masked)
        // every K buffer, and the V tiles of the first pair of iterations (see below)
#pragma unroll
        for (int g = 0; g < NSTAGE; ++g) load_k(g);
#pragma unroll
        for (int g = 0; g < NSTAGE / 2; ++g) load_v(g);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();

        f32x16_t sA[2], sB[2];
        i32x8_t pA = {}, pB = {};
        Soft sm;
        auto finish_softmax = [&]() {
            if (__builtin_amdgcn_ballot_w64(sm.alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) w.acc[dt][r] *= sm.alpha;
                // only element 0 of the row sums is read; the others may drift.  The lane's row sum
                // belongs to its partner's query, so it takes the partner's factor.
                w.lacc[0] *= from_lane(rowsum_partner(lane), sm.alpha);
            }
        };
        stream<false, true, false>(w, ad, vbuf(0), kbuf(0), pB, sA, sA, pB, sm);  // S_0 -> sA
        mask(sA, valid_of(0));
        softmax_all(w, sm, sA, pA);  // P_0 -> pA
        finish_softmax();
        __syncthreads();

        // Iteration t: P.V of tile t-1 (V_{t-1}), the softmax of tile t, the scores of tile t+1
        // (K_{t+1}).  With P = t mod NSTAGE a compile-time constant, the buffers it reads are
        // constants, which fold into the LDS reads' offset fields.
        // (always inlined: as calls, the register arrays they touch would go to scratch)
        auto body = [&](auto phase, int t, i32x8_t& p_prev, i32x8_t& p_cur, f32x16_t(&s_cur)[2],
                        f32x16_t(&s_next)[2]) __attribute__((always_inline)) {
            constexpr int P = decltype(phase)::value;
            constexpr unsigned k_next = ((P + 1) % NSTAGE) * TILE;                     // K_{t+1}
            constexpr unsigned v_prev = (NSTAGE + (P + NSTAGE - 1) % NSTAGE) * TILE;  // V_{t-1}
            if (t == 0) {
                stream<false, true, false>(w, ad, v_prev, k_next, p_prev, s_cur, s_next, p_cur, sm);
            } else {
                stream<true, true, true>(w, ad, v_prev, k_next, p_prev, s_cur, s_next, p_cur, sm);
                finish_softmax();
            }
            if (t + 1 < nkt) mask(s_next, valid_of(t + 1));
        };
        // Iterations run in pairs (t, t+1), t odd, with one barrier per pair: waves may drift apart
        // within a pair.  A pair reads K_{t+1}, K_{t+2}, V_{t-1}, V_t; at its start the loading
        // waves issue the next pair's tiles K_{t+3}, K_{t+4}, V_{t+1}, V_{t+2}, into the buffers of
        // K_{t-1}, K_t, V_{t-3}, V_{t-2}, all last read before the previous barrier; at its end
        // they wait for those loads, and the barrier publishes them.
        static_assert(NSTAGE == 4, "two pairs of iterations cycle through the four buffers");
        auto pair = [&](auto ph0, auto ph1, int t) __attribute__((always_inline)) {
            load_k(t + 3);
            load_k(t + 4);
            load_v(t + 1);
            load_v(t + 2);
            body(ph0, t, pA, pB, sB, sA);                 // odd t: P_{t-1} in pA, S_t in sB
            if (t + 1 < nkt) body(ph1, t + 1, pB, pA, sA, sB);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __syncthreads();
        };
        using Ph0 = std::integral_constant<int, 0>;
        using Ph1 = std::integral_constant<int, 1>;
        using Ph2 = std::integral_constant<int, 2>;
        using Ph3 = std::integral_constant<int, 3>;
        body(Ph0{}, 0, pB, pA, sA, sB);  // scores S_1 -> sB
        __syncthreads();                 // K_1's buffer is refilled by the first pair
        int t = 1;
        for (; t + 3 < nkt; t += 4) {
            pair(Ph1{}, Ph2{}, t);
            pair(Ph3{}, Ph0{}, t + 2);
        }
        // t = 1 mod 4 here: at most three more iterations
        if (t < nkt) {
            pair(Ph1{}, Ph2{}, t);
            t += 2;
        }
        if (t < nkt) {
            pair(Ph3{}, Ph0{}, t);
            t += 2;
        }
        if (nkt & 1)
            stream<true, false, false>(w, ad, vbuf(nkt - 1), kbuf(0), pA, sA, sA, pB, sm);
        else
            stream<true, false, false>(w, ad, vbuf(nkt - 1), kbuf(0), pB, sA, sA, pA, sm);

        // epilogue: O = acc * v_descale / l, LSE = ln2 (m + log2 l - kPShift)
        const float l_tot = from_lane(rowsum_partner(lane), w.lacc[0]);
        const float inv_l = ar.v_descale / l_tot;
        const float lse2 = w.m_run + log2f(l_tot) - kPShift;
        if (qrow < ar.Sq) {
            if (sk_slot_ < 0 && ar.o_bf16) {
                unsigned short* op = (unsigned short*)ar.o + b * ar.os.b + h * ar.os.h + (int64_t)qrow * ar.os.s;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int d = 32 * dt + 8 * r4 + 4 * hi;
                        u32x2_t wd;
                        wd[0] = pack_bf16(w.acc[dt][4 * r4] * inv_l, w.acc[dt][4 * r4 + 1] * inv_l);
                        wd[1] = pack_bf16(w.acc[dt][4 * r4 + 2] * inv_l, w.acc[dt][4 * r4 + 3] * inv_l);
                        *(u32x2_t*)(op + d) = wd;
                    }
                if (hi == 0) ar.lse[(int64_t)bh * ar.Sq + qrow] = lse2 * kLn2;
            } else {
                // the final fp32 output, or a tail segment's fp32 partial and LSE in its slot
                float* op;
                float* lp;
                if (sk_slot_ < 0) {
                    op = (float*)ar.o + b * ar.os.b + h * ar.os.h + (int64_t)qrow * ar.os.s;
                    lp = ar.lse + (int64_t)bh * ar.Sq + qrow;
                } else {
                    const int64_t r = (int64_t)sk_slot_ * kSkRows + (qrow - qt * BQ);
                    op = ar.sk_o + r * D;
                    lp = ar.sk_lse + r;
                }
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int d = 32 * dt + 8 * r4 + 4 * hi;
                        *(u32x4_t*)(op + d) = u32x4_t{__float_as_uint(w.acc[dt][4 * r4] * inv_l),
                                                      __float_as_uint(w.acc[dt][4 * r4 + 1] * inv_l),
                                                      __float_as_uint(w.acc[dt][4 * r4 + 2] * inv_l),
                                                      __float_as_uint(w.acc[dt][4 * r4 + 3] * inv_l)};
                    }
                if (hi == 0) *lp = lse2 * kLn2;
            }
        }
    }
}

}  // namespace

int fp8_key_tiles(int Skv) { return (Skv + BK - 1) / BK; }

hipError_t launch_fp8_pack_v(const Fp8Args& a, hipStream_t stream) {
    const int n_kt = fp8_key_tiles(a.Skv);
    const int64_t blocks = (int64_t)a.B * a.H * n_kt;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fp8_pack_v_kernel, dim3((unsigned)blocks), dim3(PACK_T), 0, stream, a, n_kt);
    return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream) {
    const int n_qt = (a.Sq + BQ - 1) / BQ;
    const int n_kt = fp8_key_tiles(a.Skv);
    const int64_t n_q = (int64_t)a.B * a.H * n_qt;
    if (n_q <= 0 || n_kt <= 0) return hipSuccess;
    int64_t blocks = n_q;
    if (a.sk_wgs != 0) {
        // a stream-K tail: every run of its units must stay within two query tiles
        if (a.n_dp < 0 || a.n_dp >= n_q || a.sk_wgs <= n_q - a.n_dp || !a.sk_o || !a.sk_lse)
            return hipErrorInvalidValue;
        if (a.sk_parts < 0 || (a.sk_parts > 0 && (a.sk_parts > n_kt || (int64_t)a.sk_parts * (n_q - a.n_dp) != a.sk_wgs)))
            return hipErrorInvalidValue;
        blocks = (int64_t)a.n_dp + a.sk_wgs;
    }
    if (blocks > 0x7FFFFFFF || a.persist < 0 || (a.persist > 0 && !a.wq)) return hipErrorInvalidValue;
    // per device: the kernel's dynamic LDS limit has been raised (an atomic flag, so that
    // first calls from several threads are safe: each may set the attribute, which is idempotent)
    static std::atomic<bool> attr_set[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !attr_set[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute((const void*)fwd_fp8_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) attr_set[dev].store(true, std::memory_order_release);
    }
    Fp8Args ka = a;
    int64_t grid = blocks;
    if (a.persist > 0 && blocks > a.persist) {
        e = launch_wq_clear(a.wq, stream);  // the queues start empty
        if (e != hipSuccess) return e;
        grid = a.persist;
    } else {
        ka.persist = 0;  // one round: every item has its own workgroup
    }
    hipLaunchKernelGGL(fwd_fp8_kernel, dim3((unsigned)grid), dim3(NT), LDS_BYTES, stream, ka, n_qt, n_kt);
    return hipGetLastError();
}

}  // namespace lsdit
