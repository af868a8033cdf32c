// Chunk attention forward, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Computes, for one chunk of keys, O = softmax(scale * Q K^T) V and the
// per-row natural-log LSE, blockwise over key tiles with an online softmax
// (running max, running sum, rescale) — the evaluation that lets a rank fold
// in key/value blocks one at a time without materialising the full K and V
// (NVIDIA Technical Blog "Scaling AI Inference Across Multiple GPUs Using
// NVIDIA TensorRT with Multi-Device Inference Support", section "Ring
// Attention").
//
// Work decomposition: one workgroup = 8 waves = 256 query rows of one head,
// one workgroup per CU (two waves per SIMD).  When the query tiles leave the
// last round of CUs part-full, that round's work is spread evenly instead
// (the balanced tail): each of its workgroups takes an equal run of (query
// tile, key tile) units and writes fp32 partials that a fix-up kernel merges.
//  * each wave owns 32 query rows; its Q rows stay in VGPRs for the whole
//    key loop as the B operand of v_mfma_f32_32x32x16_bf16;
//  * scores are computed transposed, S^T = K Q^T, so every lane holds 32
//    scores of ONE query row (lanes l and l+32 share a row); row max and row
//    sum are in-lane plus one permlane32 swap;
//  * P^T leaves the accumulator registers as bf16 and is fed directly as the
//    B operand of O^T += V^T P^T.  The MFMA k index is a relabelling of the
//    keys, so V^T is read from the row-major V tile with ds_read_b64_tr_b16
//    at the matching key rows;
//  * per 64-key tile t a wave runs one hand-ordered stream of MFMA slots:
//    the P.V MFMAs of tile t-1, then the score MFMAs of tile t+1.  Each slot
//    also issues the LDS read of the operand kPrefetch slots ahead (the last
//    slots those of the next stream, so no stream starts on an LDS wait), and the
//    slots carry a fixed share of the softmax of tile t: the max tree, then
//    the probabilities as a three-stage software pipeline (FMA, exp, pack
//    and sum in consecutive slots), so no slot holds a dependent VALU chain
//    that would stall the wave's next MFMA.  The scores of alternate tiles
//    sit in two register buffers, so the softmax spreads over all the slots
//    while the score MFMAs fill the other buffer.  Scheduling barriers pin
//    this order: left to itself the compiler moves each LDS read next to its
//    MFMA (exposing the LDS latency on every MFMA) and bunches the MFMAs
//    apart from the VALU;
//  * K/V tiles of 64 rows go HBM -> LDS directly (buffer loads with the LDS
//    destination) into four buffers each (K in the low 64 KiB, V above), K
//    issued three iterations and V two iterations before use, and the key
//    loop is unrolled by four, so every LDS read names its buffer by a
//    compile-time offset; loads go through buffer resources whose out-of-range
//    rows read as zero (and are masked); waves 0-3 issue all of them (the
//    older wave of each SIMD, which otherwise idles at the loop barrier);
//    LDS rows are XOR swizzled in 16-byte chunks so both the row reads of K
//    and the transposed reads of V are free of bank conflicts;
//  * exponentials are base 2 with scale*log2(e) folded into one FMA; the
//    running output is rescaled only when a row maximum grows by more than
//    64 (log2 units) past the one it was last rescaled to, and the weights,
//    taken against that maximum plus 64, stay at most 1.
// Workgroups are remapped so that each XCD (workgroups are dealt to the 8
// XCDs round-robin) runs consecutive query tiles of the same head, which
// then share K/V tiles in that XCD's L2.
// Long launches run persistent: one workgroup per CU, taking items (whole
// query tiles, then the tail's runs) from per-XCD work queues, so that the
// XCDs, whose clocks differ by several percent, end together: a fast XCD
// takes a slow one's remaining whole tiles first, then runs from any queue.
#include "kernels.h"

#include <atomic>
#include <math.h>
#include <stddef.h>

#include <type_traits>

namespace lsdit {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;
// Kernel arguments seen through the constant address space (scalar loads).
template <class T>
using kernarg_t = __attribute__((address_space(4))) const T;

constexpr float kLn2 = 0.69314718055994531f;
// Lazy-rescale threshold, log2 units.  bf16 P and the fp32 sums have 8-bit exponents, so a
// weight taken 64 below the reference is still a normal number with its full mantissa; only
// weights under 2^-62 times the row max's own could become subnormal (flushed): a relative
// change far under the fp32 rounding of the sums, even over 10^5 keys.  A large threshold makes
// the rescale (a VALU pass over the output accumulators, which costs the co-issued MFMA wave
// cycles) rare: after a row's first tile its reference moves only for a tile whose row max lies
// more than 64 (log2 units, a factor 2^64 in weight) above the max the reference was set from.
constexpr float kRescale = 64.0f;
constexpr int kPrefetch = 4;      // MFMA operands read this many slots ahead
// The softmax of a tile runs over every slot of the stream (its scores in a second register
// buffer, so the score MFMAs of the next tile may overwrite the other one meanwhile), rather
// than over the P.V slots only: half the VALU work next to each MFMA.
constexpr bool kSpread = true;

template <int D>
struct Cfg {
    static constexpr int NW = 8;                  // waves per workgroup
    static constexpr int NT = NW * 64;            // threads per workgroup
    static constexpr int BQ = 32 * NW;            // query rows per workgroup
    static constexpr int BK = 64;                 // keys per tile
    static constexpr int CH = D / 8;              // 16-byte chunks per row
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int TILE_BYTES = BK * ROW_BYTES;
    static constexpr int NSTAGE = 4;                        // LDS buffers per tensor (loop unrolled by NSTAGE)
    static constexpr int V_REGION = NSTAGE * TILE_BYTES;    // K buffers below, V buffers from here
    static constexpr int ITEM_ADDR = 2 * NSTAGE * TILE_BYTES;  // the next item, broadcast to the waves
    static constexpr int LDS_BYTES = ITEM_ADDR + 16;
    static constexpr int ROWS_PER_BLK = 64 / CH;            // rows one wave-wide 1 KiB load covers
    static constexpr int BLKS = BK / ROWS_PER_BLK;          // 1 KiB blocks per tile
    // Waves 0-3 (one per SIMD) issue all tile loads.  Each SIMD runs wave w and wave w+4,
    // and the older one (w) wins issue arbitration and reaches the loop barrier first, so
    // its idle time there absorbs the load issue that would otherwise delay wave w+4.
    static constexpr int LOADERS = NW / 2;
    static constexpr int BLKS_PER_WAVE = BLKS / LOADERS;
    static_assert(BLKS % NW == 0, "tile must split evenly over the waves");
    static constexpr int N_PV = (D / 32) * 4;               // P.V slots: (ks, dt), dt fastest
    static constexpr int N_S = (D / 16) * 2;                // score slots: (kk, kb), kb fastest
};

// XOR swizzles of the 16-byte chunk index within a row (bijections on 0..CH-1).
// K: lanes reading consecutive rows at one chunk land in distinct bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    if constexpr (D == 128) return row & 15;
    else return (row & 7) ^ ((row >> 3) & 1);
}
// V: a wave's transposed reads touch 4 consecutive rows (row & 3) and, per
// 16 lanes, two neighbouring chunks; these masks spread them over the banks.
template <int D>
__device__ __forceinline__ int v_swz(int row) {
    const int s0 = row & 1, s1 = (row >> 1) & 1;
    if constexpr (D == 128) return 10 * s0 + 4 * s1;
    else return 2 * s0 + 4 * s1;
}

// Workgroups are dispatched to the 8 XCDs round-robin; give XCD x a contiguous
// range of logical tiles so its concurrently resident workgroups share K/V.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    constexpr int X = 8;
    const int q = n / X, r = n % X;
    const int xcd = bid % X, slot = bid / X;
    return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// A weight 2^x, x <= 0 (so at most 1).  The clamp to [0, 1] folds into the exponential
// (v_exp_f32 ... clamp) and maps NaN to 0: a NaN query row (every score NaN) then adds nothing
// to the row-sum MFMA, whose zero entries would otherwise carry the NaN into the sum of the
// query sharing its MFMA column.  The NaN still reaches the row's own output, through its
// reference and scale factor (see the lazy rescale).
__device__ __forceinline__ float weight_exp2(float x) {
    return __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x), 0.f, 1.f);
}

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

// IEEE maximum (NaN-propagating): one v_maximum3_f32 per call, on raw MFMA results too.  (The
// NaN-ignoring fmaxf needs its inputs quieted first, one more instruction per input that is not
// already the result of a max.)  Row maxima of scores are the only use; a NaN score makes its
// row NaN either way.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Row sums on the matrix unit.  A lane's P^T fragment of one 16-key step (8 bf16: query
// l % 32, keys of half l / 32) is also a valid B operand of v_mfma_f32_16x16x32_bf16, which
// reads lane l as column l % 16 and k group l / 16: there the four lane groups hold queries
// 0-15 and 16-31 of both key halves.  An A operand that is 1 where its k group's parity equals
// bit 3 of its row sums, into rows 0-7 of column n, both key halves of query n, and into rows
// 8-15 those of query n + 16.  The output puts rows 4 (l / 16) .. +3 of column l % 16 in lane
// l, so lane l receives the row sum of query (l % 16) + 16 (l >= 32): its own query l % 32 for
// lanes 0-15 and 48-63, the query of lane l - 16 (l + 16) for lanes 32-47 (16-31).  The sums are
// those of the bf16 probabilities P.V uses, in fp32.
__device__ __forceinline__ bf16x8_t rowsum_a_operand(int lane) {
    const __bf16 v = ((lane >> 4) & 1) == ((lane & 15) >> 3) ? (__bf16)1.0f : (__bf16)0.0f;
    return bf16x8_t{v, v, v, v, v, v, v, v};
}
// The lane whose value belongs to the query lane l holds a row sum of (and the reverse).
__device__ __forceinline__ int rowsum_partner(int lane) {
    return lane < 16 || lane >= 48 ? lane : (lane < 32 ? lane + 16 : lane - 16);
}
__device__ __forceinline__ float from_lane(int src, float x) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(x)));
}

// Buffer resource: base, no stride, num_records bytes; reads at or past num_records return
// zeros.
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
// Resource of one tile: the bytes [off, end) of a head's rows, rebased to off (empty when off >=
// end).  The raw-buffer range check applies to the per-lane offset, not to a scalar offset, so
// every tile gets a resource of its own: the rows of a last partial tile past the tensor's end,
// and the tiles prefetched past the last chunk, then read as zeros instead of whatever memory
// follows the tensor.  Wave-uniform, so all of it is scalar arithmetic.
__device__ __forceinline__ Rsrc tile_rsrc(const void* base, int off, int end) {
    return make_rsrc((const unsigned char*)base + off, off < end ? end - off : 0);
}

// NB wave-wide 16-byte-per-lane loads into consecutive 1 KiB LDS blocks at LDS byte address
// dst.  Written as assembly on purpose: for the builtin form the compiler assumes that any
// later LDS read may read what the load writes, and waits for the load to land before the
// next ds_read — which would expose the whole load latency in every iteration of the key
// loop.  Here the kernel orders these writes itself (an explicit vmcnt wait, then a
// barrier, before any wave reads the buffer).  The loads have no register results, so
// nothing the compiler allocates is written while they are in flight.  M0 holds the LDS
// address (an operand of the statement, so the compiler sets it and knows it is used);
// one wait state separates its write from the load.
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

// Position in the key-tile sequence of a chunk list: the tile that starts at key row `row`
// of chunk c, whose rows end at `end`.  Wave-uniform (scalar registers).  Chunk c's start row
// and length sit in lane c of two vector registers and are read with readlane, so walking
// needs no memory access.  Past the last chunk the walk stays at row `past` (beyond the
// tensor, where the buffer loads read zeros).
template <int BK>
struct TileWalk {
    int c, row, end;

    __device__ __forceinline__ void enter(int ci, int n_chunks, int v_row, int v_len, int past) {
        c = ci;
        if (ci < n_chunks) {
            row = __builtin_amdgcn_readlane(v_row, ci);
            end = row + __builtin_amdgcn_readlane(v_len, ci);
        } else {
            row = past;
            end = past + BK;
        }
    }
    __device__ __forceinline__ void next(int n_chunks, int v_row, int v_len, int past) {
        row += BK;
        if (row >= end) {
            // keeps the chunk-table reads (VALU readlanes) behind the branch: hoisted, they
            // would run on every tile
            asm volatile("");
            enter(c + 1, n_chunks, v_row, v_len, past);
        }
    }
    __device__ __forceinline__ int valid() const { return end - row; }  // >= BK: a full tile
    // Tile g of the sequence (a scalar walk over the chunks' tile counts).
    __device__ __forceinline__ void seek(int g, int n_chunks, int v_row, int v_len, int past) {
        int ci = 0;
        for (; ci < n_chunks; ++ci) {
            const int nt = (__builtin_amdgcn_readlane(v_len, ci) + BK - 1) / BK;
            if (g < nt) break;
            g -= nt;
        }
        enter(ci, n_chunks, v_row, v_len, past);
        if (ci < n_chunks) row += g * BK;
    }
};

// Per-wave state of the key loop.
template <int D>
struct Wave {
    f32x16_t acc[D / 32];  // O^T accumulators
    bf16x8_t qf[D / 16];   // Q rows, MFMA B operands
    float m_run;           // softmax reference (scaled, log2 domain): a row max + kRescale
    float m_max;           // the row's largest raw score so far
    f32x4_t lacc;          // row sums (every element; lanes 16-47 hold their partner's query)
    bf16x8_t rs_a;         // A operand of the row-sum MFMA
    unsigned k_lane[D / 16];  // per-lane LDS read address of K operand kk in K buffer 0
    unsigned v_lane[D / 32];  // per-lane LDS read address of V^T operand dt in V buffer 0
    float c;               // scale * log2(e)
};

// Element f (0..31) of a lane's score tile (f is a compile-time constant after unrolling).
__device__ __forceinline__ float sel_f(const f32x16_t (&s)[2], int f) { return s[f >> 4][f & 15]; }

// Last slot of the softmax pipeline's first stage (see pair_slot): with kSpread the pipeline
// ends on the stream's last slot; otherwise on the last P.V slot + 2, so that every score is
// read before the score MFMAs overwrite it.
template <int D>
__host__ __device__ constexpr int last_a_slot() {
    return kSpread ? Cfg<D>::N_PV + Cfg<D>::N_S - 3 : Cfg<D>::N_PV - 1;
}

// Softmax state carried across the slots of one stream.
struct Soft {
    float mt[11];           // partial maxima
    float m0, m1;           // row max of each half of the wave
    float m_new, alpha;
    float x[16][2];         // stage A results (scaled, shifted scores)
    float e[16][2];         // stage B results (probabilities)
};

// Positions of the softmax work in a stream.  The max tree takes slots 0..4; probability
// pair J (scores 2J, 2J+1 -> word J%4 of p[J/4]) then runs as a 3-stage pipeline: A (two
// FMAs) at slot a(J), B (two exps) at a(J)+1, C (pack, sums) at a(J)+2, with a(J) spread
// evenly over 5..LA.  So every slot's VALU ops are independent of each other (a dependent
// chain inside a slot would hold up the wave's next MFMA, since a wave issues in order),
// and with LA the last P.V slot, all reads of the scores finish before the score MFMAs of
// the next tile overwrite them.
__host__ __device__ constexpr int pair_slot(int j, int la) { return 5 + j * (la - 4) / 16; }

// One probability buffer serves both the P.V of tile t-1 (reading it) and the softmax of tile t
// (writing it): P.V reads word group ks of P^T in slots ks*(D/32) .. ks*(D/32) + D/32 - 1, and
// the first pack into group ks (pair 4ks's stage C) comes in a later slot.
template <int D>
__host__ __device__ constexpr bool one_p_buffer_suffices() {
    for (int ks = 0; ks < 4; ++ks)
        if (pair_slot(4 * ks, last_a_slot<D>()) + 2 <= ks * (D / 32) + D / 32 - 1) return false;
    return true;
}
static_assert(one_p_buffer_suffices<128>() && one_p_buffer_suffices<64>(), "probability buffer reused too early");

// Empty asm statements (register operands only) pin a stage's results to its slot: the
// scheduling barriers order instructions, but pure arithmetic could still be sunk towards
// its use.  Only results are pinned: pinning an input read out of a live score vector would
// make the compiler copy it first (one move per input).
__device__ __forceinline__ void pin(float& a, float& b) { asm volatile("" : "+v"(a), "+v"(b)); }

template <int POS, int LA, int J = 0>
__device__ __forceinline__ void pair_stages(float c, Soft& sm, const f32x16_t (&s)[2], u32x4_t (&p)[4]) {
    if constexpr (J < 16) {
        constexpr int a = pair_slot(J, LA);
        if constexpr (POS == a) {
            const float x0 = s[J >> 3][2 * (J & 7)], x1 = s[J >> 3][2 * (J & 7) + 1];
            sm.x[J][0] = __builtin_fmaf(x0, c, -sm.m_new);
            sm.x[J][1] = __builtin_fmaf(x1, c, -sm.m_new);
            pin(sm.x[J][0], sm.x[J][1]);
        } else if constexpr (POS == a + 1) {
            sm.e[J][0] = weight_exp2(sm.x[J][0]);
            sm.e[J][1] = weight_exp2(sm.x[J][1]);
            pin(sm.e[J][0], sm.e[J][1]);
        } else if constexpr (POS == a + 2) {
            unsigned word = pack_bf16(sm.e[J][0], sm.e[J][1]);
            asm volatile("" : "+v"(word));
            p[J >> 2][J & 3] = word;
        }
        pair_stages<POS, LA, J + 1>(c, sm, s, p);
    }
}

// The share of the softmax of s that stream position POS carries.
template <int D, int POS>
__device__ __forceinline__ void softmax_slot(Wave<D>& w, Soft& sm, const f32x16_t (&s)[2], u32x4_t (&p)[4]) {
    if constexpr (POS == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.mt[i] = max3(sel_f(s, 3 * i), sel_f(s, 3 * i + 1), sel_f(s, 3 * i + 2));
    } else if constexpr (POS == 1) {
#pragma unroll
        for (int i = 4; i < 8; ++i) sm.mt[i] = max3(sel_f(s, 3 * i), sel_f(s, 3 * i + 1), sel_f(s, 3 * i + 2));
    } else if constexpr (POS == 2) {
        sm.mt[8] = max3(sel_f(s, 24), sel_f(s, 25), sel_f(s, 26));
        sm.mt[9] = max3(sel_f(s, 27), sel_f(s, 28), sel_f(s, 29));
        // every raw score enters through a three-input max: 32 scores in 16 v_maximum3
        sm.mt[10] = max3(sel_f(s, 30), sel_f(s, 31), sm.mt[0]);
        sm.mt[1] = max3(sm.mt[1], sm.mt[2], sm.mt[3]);
    } else if constexpr (POS == 3) {
        const float mx = max3(max3(sm.mt[1], sm.mt[4], sm.mt[5]), max3(sm.mt[6], sm.mt[7], sm.mt[8]),
                              vmax(sm.mt[9], sm.mt[10]));
        half_pair(mx, sm.m0, sm.m1);
    } else if constexpr (POS == 4) {
        // Lazy rescale.  A row's reference r sits kRescale (log2 units) above the row max it
        // was last moved to, and moves only when a tile's row max m exceeds it, or is NaN: to
        // m + kRescale.  So every weight 2^(s c - r) is at most 1 (at most 2^-kRescale right
        // after a move), O and l share the reference (consistent), and LSE = r + log2 l.  A NaN
        // row max (a NaN score) moves the reference to NaN, which makes the rescale factor and
        // so the row's output and LSE NaN.  Lanes l and l+32 hold the same row and agree.  The
        // test runs on the running max (at most r before this tile, so it exceeds r exactly
        // when this tile's max does, and then equals it): one three-input max keeps it.
        w.m_max = max3(w.m_max, sm.m0, sm.m1);
        const float m_tile = w.m_max * w.c;
        sm.m_new = !(m_tile <= w.m_run) ? m_tile + kRescale : w.m_run;
        sm.alpha = fast_exp2(w.m_run - sm.m_new);
        w.m_run = sm.m_new;
    }
    pair_stages<POS, last_a_slot<D>()>(w.c, sm, s, p);
}

// All softmax positions in order (for a tile whose softmax runs on its own).
template <int D, int POS = 0>
__device__ __forceinline__ void softmax_all(Wave<D>& w, Soft& sm, const f32x16_t (&s)[2], u32x4_t (&p)[4]) {
    if constexpr (POS < last_a_slot<D>() + 3) {
        softmax_slot<D, POS>(w, sm, s, p);
        softmax_all<D, POS + 1>(w, sm, s, p);
    }
}

// One MFMA operand (16 bytes) of stream slot SLOT.  vb / kb are this lane's read offsets
// with the buffer's LDS offset OR-ed in (buffers are tile-aligned, so the swizzled low bits
// are untouched); XOR-ing the slot constant into that loop-variant value keeps the compiler
// from hoisting a table of loop-invariant addresses out of the key loop (and spilling it).
template <int D, int SLOT>
__device__ __forceinline__ u32x4_t read_opnd(const Wave<D>& w, unsigned vb, unsigned kb_) {
    using C = Cfg<D>;
    // vb and kb_ are the buffers' byte offsets within the V and K regions: in the unrolled key
    // loop compile-time constants, so each address is a per-lane register plus the read's
    // offset field
    if constexpr (SLOT < C::N_PV) {
        constexpr int ks = SLOT / (D / 32), dt = SLOT % (D / 32);
        const unsigned a = w.v_lane[dt] + vb + 16 * ks * C::ROW_BYTES;
        const u32x2_t lo = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(size_t)a));
        const u32x2_t hi = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(size_t)(a + 8 * C::ROW_BYTES)));
        return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    } else {
        constexpr int sl = SLOT - C::N_PV, kk = sl >> 1, kb = sl & 1;
        return *(const lds_u32x4_t*)(size_t)(w.k_lane[kk] + kb_ + kb * 32 * C::ROW_BYTES);
    }
}

// Slot SLOT of a stream (see stream()), then the following slots.
template <int D, bool DO_PV, bool DO_S, bool DO_SM, bool NEXT, int SLOT>
__device__ __forceinline__ void stream_slots(Wave<D>& w, unsigned vb, unsigned kb_, unsigned vb_next, bool bar,
                                             u32x4_t (&ring)[kPrefetch], const u32x4_t (&p_prev)[4],
                                             const f32x16_t (&s_cur)[2], f32x16_t (&s)[2], u32x4_t (&p_cur)[4],
                                             Soft& sm) {
    using C = Cfg<D>;
    constexpr int first = DO_PV ? 0 : C::N_PV;
    constexpr int last = DO_S ? C::N_PV + C::N_S : C::N_PV;
    if constexpr (SLOT < last) {
        constexpr int pos = SLOT - first;
        if constexpr (NEXT && SLOT == last - kPrefetch) {
            // the pair's barrier, before the reads of the next stream's operands: its V tile
            // may be one this pair's loads brought in (the last MFMA operands of this stream
            // are in registers by now: the barrier waits for every LDS read)
            if (bar) {
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                __syncthreads();
            }
        }
        const u32x4_t op = ring[pos % kPrefetch];
        if constexpr (SLOT < C::N_PV) {
            constexpr int ks = SLOT / (D / 32), dt = SLOT % (D / 32);
            w.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, op),
                                                                __builtin_bit_cast(bf16x8_t, p_prev[ks]), w.acc[dt],
                                                                0, 0, 0);
            // the row sums of this 16-key step ride on the step's last P.V slot
            if constexpr (dt == D / 32 - 1)
                w.lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w.rs_a, __builtin_bit_cast(bf16x8_t, p_prev[ks]),
                                                                 w.lacc, 0, 0, 0);
        } else {
            constexpr int sl = SLOT - C::N_PV, kk = sl >> 1, kb = sl & 1;
            if constexpr (kk == 0) {
                const f32x16_t zero = {};
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, op), w.qf[kk], zero, 0,
                                                                0, 0);
            } else {
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, op), w.qf[kk], s[kb], 0,
                                                                0, 0);
            }
        }
        if constexpr (SLOT + kPrefetch < last)
            ring[pos % kPrefetch] = read_opnd<D, SLOT + kPrefetch>(w, vb, kb_);
        else if constexpr (NEXT)  // the next stream's P.V operand SLOT + kPrefetch - last
            ring[pos % kPrefetch] = read_opnd<D, SLOT + kPrefetch - last>(w, vb_next, 0);
        if constexpr (DO_SM && pos < last_a_slot<D>() + 3) softmax_slot<D, pos>(w, sm, s_cur, p_cur);
        __builtin_amdgcn_sched_barrier(0);
        stream_slots<D, DO_PV, DO_S, DO_SM, NEXT, SLOT + 1>(w, vb, kb_, vb_next, bar, ring, p_prev, s_cur, s, p_cur,
                                                            sm);
    }
}

template <int D, bool DO_PV, int I = 0>
__device__ __forceinline__ void ring_fill(const Wave<D>& w, unsigned vb, unsigned kb_, u32x4_t (&ring)[kPrefetch],
                                          int last) {
    using C = Cfg<D>;
    constexpr int first = DO_PV ? 0 : C::N_PV;
    if constexpr (I < kPrefetch) {
        if (first + I < last) ring[I] = read_opnd<D, first + I>(w, vb, kb_);
        ring_fill<D, DO_PV, I + 1>(w, vb, kb_, ring, last);
    }
}

// One stream: P.V of the tile at LDS offset v0 (if DO_PV, with probabilities p_prev), the
// softmax of the scores in s into p_cur (if DO_SM; on the P.V slots), then the scores of the
// tile at k0 into s (if DO_S; on the later slots, after the softmax has read s).  The operand
// ring holds the MFMA operands read ahead: FILL reads the stream's first ones at its start;
// otherwise the previous stream has read them.  With NEXT the stream's last slots read the
// first operands of the next stream, a P.V stream on the V tile at v_next, and with bar (a
// wave-uniform flag) the stream takes the pair's barrier before those reads.
template <int D, bool DO_PV, bool DO_S, bool DO_SM, bool FILL, bool NEXT>
__device__ __forceinline__ void stream(Wave<D>& w, int v0, int k0, unsigned v_next, bool bar, u32x4_t (&ring)[kPrefetch],
                                       const u32x4_t (&p_prev)[4], const f32x16_t (&s_cur)[2], f32x16_t (&s)[2],
                                       u32x4_t (&p_cur)[4], Soft& sm) {
    using C = Cfg<D>;
    static_assert(!DO_SM || (DO_PV && DO_S), "the softmax needs the full stream's slots");
    static_assert(C::N_PV >= 8 && C::N_S >= 2, "stream too short for the softmax pipeline");
    constexpr int first = DO_PV ? 0 : C::N_PV;
    constexpr int last = DO_S ? C::N_PV + C::N_S : C::N_PV;
    // a read for the next stream's operand j lands in the ring entry that stream takes it from
    static_assert(!NEXT || ((last - first) % kPrefetch == 0 && C::N_PV >= kPrefetch), "ring out of step");
    const unsigned vb = v0, kb_ = k0;
    if constexpr (FILL) ring_fill<D, DO_PV>(w, vb, kb_, ring, last);
    __builtin_amdgcn_sched_barrier(0);
    stream_slots<D, DO_PV, DO_S, DO_SM, NEXT, first>(w, vb, kb_, v_next, bar, ring, p_prev, s_cur, s, p_cur, sm);
}

template <int D>
__global__ __launch_bounds__(Cfg<D>::NT, 1) void fwd_bf16_kernel(FwdArgs a, int n_qt, float c) {
    using C = Cfg<D>;
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_qtiles = a.B * a.H * n_qt;
    const int Skv = a.Skv;  // key rows of the k and v tensors
    static_assert(C::BQ == kSkRows, "stream-K slots hold one query tile");

    // ---- the chunk list: lane c holds chunk c's first row and length (read through the
    // kernel-argument pointer, so the argument array is not copied to registers first)
    const int n_chunks = a.n_chunks;
    const int* const arg_rows =
        (const int*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(FwdArgs, chunk_row));
    const int* const arg_lens =
        (const int*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(FwdArgs, chunk_len));
    const int v_row = lane < n_chunks ? arg_rows[lane] : 0;
    const int v_len = lane < n_chunks ? arg_lens[lane] : 0;
    int nkt_all = 0;  // tiles over all chunks
    for (int ci = 0; ci < n_chunks; ++ci) nkt_all += (__builtin_amdgcn_readlane(v_len, ci) + C::BK - 1) / C::BK;

    // ---- this workgroup's work: items (FwdArgs), each one or two segments (query tile, run of
    // the key-tile sequence).  A whole query tile is one segment; a tail run spans at most two
    // query tiles.  The first item is the workgroup's own index; a persistent workgroup then
    // takes items from the work queues (wq_next) until they are empty.
    // Only the item and seg are carried from one segment to the next: each iteration derives its
    // segment from them again (state kept live across the key loop would cost registers).
    int seg = 0, bid = 0;
    unsigned wq_empty = 0;  // queues found empty (thread 0's)
    for (int it = 0;; ++it) {
        // the arguments, read through a pointer the compiler cannot follow: so their loads stay
        // in the iteration rather than being hoisted in front of the loop and held in registers
        // across it
        const kernarg_t<FwdArgs>* ap = (const kernarg_t<FwdArgs>*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(ap));
        const kernarg_t<FwdArgs>& ar = *ap;
        const int n_whole = ar.sk_wgs == 0 ? n_qtiles : ar.n_dp;
        if (seg == 0) {
            if (it == 0) {
                bid = wg_logical((int)blockIdx.x, (int)gridDim.x, ar.wg_order);
            } else {
                if (ar.persist == 0) break;
                // thread 0 takes the next item as soon as its wave is done (the atomic's latency
                // overlaps the drain of the last item's stores) and broadcasts it through an LDS
                // word: every wave read the word's last value before the barrier that ends the
                // last segment's prologue, which thread 0 has passed since
                int* const item = (int*)(smem + C::ITEM_ADDR);
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
        // likewise the lane index: values derived from it are computed in the iteration
        int lane_it = lane;
        asm volatile("" : "+v"(lane_it));
        const int hi_it = lane_it >> 5;
        int sk_slot_ = -1, tile, g_first, nkt;
        if (bid < n_whole) {
            if (seg > 0) {
                seg = 0;
                continue;
            }
            tile = xcd_remap(bid, n_whole);
            g_first = 0;
            nkt = nkt_all;
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
                const int n_tail = n_qtiles - ar.n_dp, p = sk_w / n_tail;
                tile = ar.n_dp + sk_w % n_tail;
                g_first = (int)((int64_t)nkt_all * p / ar.sk_parts);
                nkt = (int)((int64_t)nkt_all * (p + 1) / ar.sk_parts) - g_first;
                sk_slot_ = sk_w;
            } else {
                const int64_t U = (int64_t)(n_qtiles - ar.n_dp) * nkt_all;
                const int64_t u0 = sk_start(U, sk_w, ar.sk_wgs), u1 = sk_start(U, sk_w + 1, ar.sk_wgs);
                // segment 0 runs to the end of u0's query tile (or to u1), segment 1 from there to u1
                const int64_t cut = (u0 / nkt_all + 1) * nkt_all;
                const int64_t s0 = seg == 0 ? u0 : cut, s1 = seg == 0 ? (u1 < cut ? u1 : cut) : u1;
                if (seg > 1 || s0 >= s1) {
                    seg = 0;
                    continue;
                }
                sk_slot_ = sk_slot(sk_w, seg, (int)(s0 / nkt_all), ar.sk_wgs);
                tile = ar.n_dp + (int)(s0 / nkt_all);
                g_first = (int)(s0 % nkt_all);
                nkt = (int)(s1 - s0);
            }
        }
        // wave-uniform: the 64-bit divisions above run on the vector unit, and left there the
        // key loop's control flow derived from these would become per-lane
        tile = __builtin_amdgcn_readfirstlane(tile);
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
        const int bh = tile / n_qt, qt = tile % n_qt;
        const int b = bh / ar.H, h = bh % ar.H;
        const unsigned short* qp = (const unsigned short*)ar.q + b * ar.qs.b + h * ar.qs.h;
        const unsigned short* kp = (const unsigned short*)ar.k + b * ar.ks.b + h * ar.ks.h;
        const unsigned short* vp = (const unsigned short*)ar.v + b * ar.vs.b + h * ar.vs.h;

        Wave<D> w;
        w.c = c;
        w.m_run = -INFINITY;
        w.m_max = -INFINITY;
        w.lacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        w.rs_a = rowsum_a_operand(lane_it);
        asm volatile("" : "+v"(w.rs_a));  // kept in registers, not rebuilt before every use
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) w.acc[dt][r] = 0.f;

        // ---- Q fragments: B operand, lane_it holds Q[row][16kk + 8hi .. +8]
        const int qrow = qt * C::BQ + wave * 32 + (lane_it & 31);
        const int qrow_c = qrow < ar.Sq ? qrow : ar.Sq - 1;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            w.qf[kk] = *(const bf16x8_t*)(qp + (int64_t)qrow_c * ar.qs.s + 16 * kk + 8 * hi_it);

        // ---- K/V loads straight into LDS.  One wave-wide instruction fills a contiguous
        // 1 KiB block (lane_it L -> bytes 16L..16L+15); lane_it L fetches the global chunk that the
        // swizzle maps to its slot.  Offsets are per lane_it and fixed; each tile gets a resource
        // based at its first row (tile_rsrc), so rows past the tensor read zeros.
        const int k_rs = (int)(ar.ks.s * 2), v_rs = (int)(ar.vs.s * 2);  // row pitch in bytes
        const int k_end = (Skv - 1) * k_rs + D * 2, v_end = (Skv - 1) * v_rs + D * 2;  // bytes of a head's rows
        int k_goff[C::BLKS_PER_WAVE], v_goff[C::BLKS_PER_WAVE];
#pragma unroll
        for (int i = 0; i < C::BLKS_PER_WAVE; ++i) {
            const int blk = wave * C::BLKS_PER_WAVE + i;
            const int row = blk * C::ROWS_PER_BLK + lane_it / C::CH, slot = lane_it % C::CH;
            k_goff[i] = row * k_rs + (slot ^ k_swz<D>(row)) * 16;
            v_goff[i] = row * v_rs + (slot ^ v_swz<D>(row)) * 16;
        }
        // The kernel declares no static LDS, so its dynamic block (smem) starts at LDS address 0
        // and every LDS access below is a plain byte address; a CPU test checks that the built
        // kernel has no static LDS.  (Pointer arithmetic on smem instead costs one add per
        // address: the block's address is a link-time constant the compiler cannot fold.)
        (void)smem;
        constexpr unsigned lds_base = 0;
        // Offsets of tile t's buffers within the K region (LDS address 0) and the V region (LDS
        // address V_REGION)
        auto kbuf = [&](int t) { return (unsigned)((t % C::NSTAGE) * C::TILE_BYTES); };
        auto vbuf = [&](int t) { return (unsigned)((t % C::NSTAGE) * C::TILE_BYTES); };
        // Three walks over the tile sequence: the next K tile to load (tile t + NSTAGE during
        // iteration t), the next V tile to load (tile t + NSTAGE - 2) and the next tile to mask
        // (tile t + 1).  Tile g of the sequence goes into buffer g mod NSTAGE.
        TileWalk<C::BK> wk, wv, wm;
        wk.seek(g_first, n_chunks, v_row, v_len, Skv);
        wv = wk;
        wm = wk;
        auto load_k = [&](int g) {
            if (wave < C::LOADERS)
                lds_dma<C::BLKS_PER_WAVE>(tile_rsrc(kp, wk.row * k_rs, k_end),
                                          lds_base + kbuf(g) + wave * C::BLKS_PER_WAVE * 1024, k_goff);
            wk.next(n_chunks, v_row, v_len, Skv);
        };
        auto load_v = [&](int g) {
            if (wave < C::LOADERS)
                lds_dma<C::BLKS_PER_WAVE>(tile_rsrc(vp, wv.row * v_rs, v_end),
                                          lds_base + C::V_REGION + vbuf(g) + wave * C::BLKS_PER_WAVE * 1024, v_goff);
            wv.next(n_chunks, v_row, v_len, Skv);
        };
        auto next_valid = [&]() {  // valid keys of the next tile to mask
            const int valid = wm.valid();
            wm.next(n_chunks, v_row, v_len, Skv);
            return valid;
        };

        // ---- per-lane_it LDS read addresses in buffer 0 of each region.  Each swizzle XOR only
        // touches chunk-index bits that the operand index sets independently, so the operand
        // index enters as an XOR with a constant (taken once here, one register per operand
        // column) and row steps, key blocks and buffers as additions (folded into the reads'
        // offset fields).
        // K operand (kb, kk): row kb*32 + (lane_it&31), chunk 2kk + hi_it  ->  k_base ^ (kk << 5)
        // (k_swz(row + 32) == k_swz(row)).
        {
            const unsigned k_base = (lane_it & 31) * C::ROW_BYTES + ((hi_it ^ k_swz<D>(lane_it & 31)) * 16);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) w.k_lane[kk] = k_base ^ (kk << 5);
        }
        // V^T operand (dt, ks, lo/hi_it): rows 16ks + 4(g>>1) + (j>>2) (+8), element columns
        // 32dt + 16(g&1) + 4(j&3)  ->  v_base ^ (dt << 6); v_swz depends on row & 3 only.
        {
            const int g = lane_it >> 4, j = lane_it & 15;
            const int v_row0 = 4 * (g >> 1) + (j >> 2);
            const int v_col0 = 16 * (g & 1) + 4 * (j & 3);
            const unsigned v_base = v_row0 * C::ROW_BYTES + (((v_col0 >> 3) ^ v_swz<D>(v_row0)) * 16) + (v_col0 & 7) * 2;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) w.v_lane[dt] = C::V_REGION + (v_base ^ (dt << 6));
        }
        // opaque to the compiler, so the offsets stay additions folded into the reads' offset
        // fields (with their bits known disjoint it may turn them into ORs computed per read)
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(w.k_lane[kk]));
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) asm volatile("" : "+v"(w.v_lane[dt]));

        // Key of accumulator element (kb, r) is kb*32 + 8(r>>2) + 4hi + (r&3); compare its
        // compile-time part against valid - 4hi, so no table of per-lane_it key indices is kept live.
        // Rows of a tile past its chunk's end (another chunk's keys, or zeros past the tensor)
        // get P = 0.
        auto mask = [&](f32x16_t(&s)[2], int valid) {
            if (valid < C::BK) {
                const int lim = valid - 4 * hi_it;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = -INFINITY;
            }
        };

        // ---- prologue.  LDS needs no clearing: every tile buffer is written whole by its loads
        // before any read (all four K buffers and V_0, V_1 here, V_2 and V_3 by the first pair of
        // iterations, before the P.V that reads them), rows past the tensor read as zeros and rows
        // past a chunk are other rows of the tensor, which the mask gives P = 0.
#pragma unroll
        for (int g = 0; g < C::NSTAGE; ++g) load_k(g);
#pragma unroll
        for (int g = 0; g < C::NSTAGE / 2; ++g) load_v(g);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q, the chunk table and the first tiles are in
        __syncthreads();

        // Scores of alternate tiles (one buffer without kSpread: the softmax of tile t then reads
        // it before the score MFMAs of tile t+1 overwrite it).
        f32x16_t sA[2], sB_own[2];
        f32x16_t(&sB)[2] = kSpread ? sB_own : sA;
        u32x4_t pp[4];  // probabilities (one buffer suffices: see one_p_buffer_suffices)
        Soft sm;
        // after the softmax of a tile: the rare rescale of the running output and row sums (the
        // latter with the factor of the query whose sum the lane_it holds)
        auto finish_softmax = [&]() {
            if (__builtin_amdgcn_ballot_w64(sm.alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) w.acc[dt][r] *= sm.alpha;
                w.lacc *= from_lane(rowsum_partner(lane_it), sm.alpha);
            }
        };
        u32x4_t ring[kPrefetch];  // MFMA operands read ahead (see stream)
        // tile 0: scores, then its softmax on its own
        stream<D, false, true, false, true, false>(w, vbuf(0), kbuf(0), 0, false, ring, pp, sA, sA, pp, sm);  // S_0
        mask(sA, next_valid());
        softmax_all<D>(w, sm, sA, pp);  // P_0
        finish_softmax();
        __syncthreads();  // every wave is done with K buffer 0 before tile NSTAGE overwrites it

        // ---- key loop.  Iteration t streams P.V of tile t-1 (V_{t-1}) with the softmax of tile t,
        // then the scores of tile t+1 (K_{t+1}).  Scores of tile nkt are computed from a stale
        // buffer and never used.  The score registers swap roles every iteration (sA <->
        // sB); the probability registers are one buffer.  With P = t mod NSTAGE a compile-time
        // constant, the buffers an iteration reads are constants, which fold into the LDS reads'
        // offset fields.  (The lambdas are always inlined: as calls, the register arrays they
        // touch would go to scratch.)
        // Each iteration's stream reads the first operands of the next one, which is the P.V of
        // tile t (V_t, buffer P): iteration t+1's stream or, after the last iteration, the final
        // P.V; bar: this stream ends its pair (takes the pair's barrier).
        auto body = [&](auto phase, int t, u32x4_t(&p_prev)[4], u32x4_t(&p_cur)[4], f32x16_t(&s_cur)[2],
                        f32x16_t(&s_next)[2], bool bar) __attribute__((always_inline)) {
            constexpr int P = decltype(phase)::value;
            constexpr unsigned k_next = ((P + 1) % C::NSTAGE) * C::TILE_BYTES;                // K_{t+1}
            constexpr unsigned v_prev = ((P + C::NSTAGE - 1) % C::NSTAGE) * C::TILE_BYTES;    // V_{t-1}
            constexpr unsigned v_cur = P * C::TILE_BYTES;                                     // V_t
            if (t == 0) {
                stream<D, false, true, false, true, true>(w, v_prev, k_next, v_cur, bar, ring, p_prev, s_cur, s_next,
                                                          p_cur, sm);
            } else {
                stream<D, true, true, true, false, true>(w, v_prev, k_next, v_cur, bar, ring, p_prev, s_cur, s_next,
                                                         p_cur, sm);
                finish_softmax();
            }
            if (t + 1 < nkt) mask(s_next, next_valid());
        };
        // Iterations run in pairs (t, t+1), t odd, with one barrier per pair: waves may drift apart
        // within a pair.  A pair reads K_{t+1}, K_{t+2}, V_{t-1}, V_t; at its start the loading
        // waves issue the next pair's tiles K_{t+3}, K_{t+4}, V_{t+1}, V_{t+2}, into the buffers of
        // K_{t-1}, K_t, V_{t-3}, V_{t-2}, all last read before the previous barrier; near its end
        // (before the last kPrefetch slots of its last stream, whose operands are in registers
        // by then) they wait for those loads, and the barrier publishes them, so that the slots
        // after it may read the next pair's first operands.
        static_assert(C::NSTAGE == 4, "two pairs of iterations cycle through the four buffers");
        auto pair = [&](auto ph0, auto ph1, int t) __attribute__((always_inline)) {
            load_k(t + 3);
            load_k(t + 4);
            load_v(t + 1);
            load_v(t + 2);
            body(ph0, t, pp, pp, sB, sA, t + 1 >= nkt);  // odd t: S_t in sB
            if (t + 1 < nkt) body(ph1, t + 1, pp, pp, sA, sB, true);
        };
        using Ph0 = std::integral_constant<int, 0>;
        using Ph1 = std::integral_constant<int, 1>;
        using Ph2 = std::integral_constant<int, 2>;
        using Ph3 = std::integral_constant<int, 3>;
        // scores S_1 -> sB; then (in the stream) a barrier: K_1's buffer is refilled by the first
        // pair
        body(Ph0{}, 0, pp, pp, sA, sB, true);
        // pairs (t, t+1) and (t+2, t+3); the last iterations may end a pair early
        for (int t = 1; t < nkt; t += 4) {
            pair(Ph1{}, Ph2{}, t);
            if (t + 2 < nkt) pair(Ph3{}, Ph0{}, t + 2);
        }
        // P.V of the last tile
        stream<D, true, false, false, false, false>(w, vbuf(nkt - 1), kbuf(0), 0, false, ring, pp, sA, sA, pp, sm);

        // ---- epilogue: normalise, LSE, fold in the running result if there is one, store (the
        // final output; or, for a stream-K segment, an fp32 partial and its LSE in the segment's
        // slot)
        const float l_tot = from_lane(rowsum_partner(lane_it), w.lacc[0]);
        const float inv_l = 1.f / l_tot;
        // The row sum adds the weights as P.V uses them, rounded to bf16, and O divides by it.
        // The LSE takes the row's largest weight unrounded: that weight, recomputed exactly as
        // the key loop computed it (no tile after the max's moved the reference: a move needs a
        // larger max), replaces its rounded value.  Where one key dominates the row, its
        // rounding (up to 2^-9 relative) would otherwise be the LSE's error.  A NaN or empty row
        // gets no correction (the clamped exponential maps NaN to 0).
        const float e_max = weight_exp2(__builtin_fmaf(w.m_max, w.c, -w.m_run));
        const float lse2 = w.m_run + log2f(l_tot + (e_max - (float)(__bf16)e_max));  // log2 domain
        if (qrow < ar.Sq) {
            // output element o = wc * acc + wr * O_run (wc = 1/l without a running result)
            float lse_out = lse2 * kLn2, wc = inv_l, wr = 0.f;
            const float* rp = nullptr;
            if (sk_slot_ < 0 && ar.run_lse) {
                const int64_t rrow = (int64_t)bh * ar.Sq + qrow;
                rp = ar.run_o + rrow * D + 4 * hi_it;
                lse_out = fold_weights(lse_out, ar.run_lse[rrow], wc, wr);
                wc *= inv_l;
            }
            // the 4 output values of accumulator group (dt, r4): d = 32 dt + 8 r4 + 4 hi .. +3
            auto vals = [&](int dt, int r4) __attribute__((always_inline)) {
                f32x4_t x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = w.acc[dt][4 * r4 + e] * wc;
                if (rp) x += wr * *(const f32x4_t*)(rp + 32 * dt + 8 * r4);
                return x;
            };
            if (sk_slot_ < 0 && ar.o_bf16) {
                unsigned short* op = (unsigned short*)ar.o + b * ar.os.b + h * ar.os.h + (int64_t)qrow * ar.os.s;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int d = 32 * dt + 8 * r4 + 4 * hi_it;
                        const f32x4_t x = vals(dt, r4);
                        u32x2_t wd;
                        wd[0] = pack_bf16(x[0], x[1]);
                        wd[1] = pack_bf16(x[2], x[3]);
                        *(u32x2_t*)(op + d) = wd;
                    }
                if (hi_it == 0) ar.lse[(int64_t)bh * ar.Sq + qrow] = lse_out;
            } else {
                float* op;
                float* lp;
                if (sk_slot_ < 0) {
                    op = (float*)ar.o + b * ar.os.b + h * ar.os.h + (int64_t)qrow * ar.os.s;
                    lp = ar.lse + (int64_t)bh * ar.Sq + qrow;
                } else {
                    const int64_t r = (int64_t)sk_slot_ * kSkRows + (qrow - qt * C::BQ);
                    op = ar.sk_o + r * D;
                    lp = ar.sk_lse + r;
                }
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) *(f32x4_t*)(op + 32 * dt + 8 * r4 + 4 * hi_it) = vals(dt, r4);
                if (hi_it == 0) *lp = lse_out;
            }
        }
    }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    using C = Cfg<D>;
    // per device: the kernel's dynamic LDS limit has been raised (an atomic flag, so that
    // first calls from several threads are safe: each may set the attribute, which is idempotent)
    static std::atomic<bool> attr_set[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !attr_set[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute((const void*)fwd_bf16_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                C::LDS_BYTES);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) attr_set[dev].store(true, std::memory_order_release);
    }
    const int n_qt = (a.Sq + C::BQ - 1) / C::BQ;
    const int64_t n_q = (int64_t)a.B * a.H * n_qt;
    int64_t n_tiles = n_q;
    if (a.sk_wgs != 0) {
        // a stream-K tail: every run of its units must stay within two query tiles
        if (a.n_dp < 0 || a.n_dp >= n_q || a.sk_wgs <= n_q - a.n_dp || !a.sk_o || !a.sk_lse)
            return hipErrorInvalidValue;
        int64_t T = 0;
        for (int c = 0; c < a.n_chunks && c < kMaxChunks; ++c) T += (a.chunk_len[c] + C::BK - 1) / C::BK;
        if (a.sk_parts < 0 || (a.sk_parts > 0 && (a.sk_parts > T || (int64_t)a.sk_parts * (n_q - a.n_dp) != a.sk_wgs)))
            return hipErrorInvalidValue;
        n_tiles = (int64_t)a.n_dp + a.sk_wgs;
    }
    if (n_tiles > 0x7FFFFFFF || a.persist < 0 || (a.persist > 0 && !a.wq)) return hipErrorInvalidValue;
    const float c = (float)((double)a.scale * 1.4426950408889634);
    FwdArgs ka = a;
    int64_t grid = n_tiles;
    if (a.persist > 0 && n_tiles > a.persist) {
        // the queues start empty (a kernel, not a memset, so that the launch can be captured)
        e = launch_wq_clear(a.wq, stream);
        if (e != hipSuccess) return e;
        grid = a.persist;
    } else {
        ka.persist = 0;  // one round: every item has its own workgroup
    }
    hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3((unsigned)grid), dim3(C::NT), C::LDS_BYTES, stream, ka, n_qt, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
    if (a.D == 128) return launch_d<128>(a, stream);
    if (a.D == 64) return launch_d<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace lsdit
