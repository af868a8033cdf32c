// Internal interface between the C-ABI host code (attn_api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace lsdit {

// Element strides of a [B, H, S, D] tensor with unit d stride.
struct Strides {
    int64_t b, h, s;
};

// One attention launch over a list of key chunks.  Pointers are device pointers.
constexpr int kMaxChunks = 64;
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    Strides qs, ks, vs;
    void* o;             // [B, H, Sq, D], o_bf16 ? bf16 : fp32, strides os
    Strides os;
    int o_bf16;
    float* lse;          // [B, H, Sq] fp32 contiguous
    int B, H, Sq, Skv, D;  // Skv: key rows of the k and v tensors
    float scale;
    // The keys attended, chunk by chunk in processing order: chunk c is rows
    // [chunk_row[c], chunk_row[c] + chunk_len[c]) of k and v.  One launch folds every chunk
    // into one online softmax, so the result is attention over the union of the chunks.
    int n_chunks;        // 1 .. kMaxChunks
    int chunk_row[kMaxChunks];
    int chunk_len[kMaxChunks];  // each > 0
    // The launch's work is a list of items, logical indices b < n_items.  Without a balanced tail
    // (sk_wgs == 0) item b is query tile xcd_remap(b, n_q) of the n_q = B*H*ceil(Sq/kSkRows) in
    // (b, h, tile) order, taken whole; n_items = n_q.
    // Balanced tail (bf16 and FP8 paths): sk_wgs > 0 makes n_items = n_dp + sk_wgs.  Items below
    // n_dp are whole query tiles (xcd_remap over the first n_dp) and write the final output.  The
    // other query tiles make U = (n_q - n_dp) * T units (query tile, key tile), T key tiles per
    // query tile; item n_dp + w is the tail's run w.  With sk_parts == 0 the runs are equal unit
    // ranges: run w takes units [sk_start(U, w, sk_wgs), sk_start(U, w + 1, sk_wgs)), at most two
    // query-tile segments because sk_wgs > n_q - n_dp makes every run at most T long, each
    // written to slot sk_slot(...).  With sk_parts == r >= 2 (sk_wgs = r * n_tail, r <= T) every
    // tail tile is cut into r parts: run w is key tiles [T p / r, T (p + 1) / r) of tail tile
    // w % n_tail, p = w / n_tail, one segment, slot w.  Each segment is written as an fp32
    // partial (normalised by its own row sum) with its natural-log LSE: row r of the query tile
    // at sk_o + slot*kSkRows*D + r*D and sk_lse + slot*kSkRows + r.  launch_sk_fixup then merges
    // the partials into the final output.
    int n_dp;
    int sk_wgs;          // runs of the tail; 0 = no tail
    int sk_parts;        // 0: runs of equal unit ranges; r >= 2: r parts per tail tile
    float* sk_o;
    float* sk_lse;
    // Dispatch.  persist == 0: one workgroup per item.  persist > 0: a persistent
    // grid of min(n_items, persist) workgroups (one per CU); workgroup g takes item g, then
    // further items from the work queues in wq (kWorkQueueWords words, zeroed before the
    // launch), until they are empty.  Results do not depend on which workgroup takes an item.
    int persist;
    unsigned* wq;
    // Running result over earlier keys (the ring's online merge done in the epilogue): when
    // run_lse is set, the output written is the LSE merge (fold_weights) of this launch's result
    // with run_o [B, H, Sq, D] fp32 contiguous / run_lse [B, H, Sq].  o and lse may alias them
    // (o fp32 with contiguous strides): every element is read before the same thread writes it.
    // Stream-K partials are written unmerged; launch_sk_fixup folds the running result in.
    const float* run_o;
    const float* run_lse;
    int wg_order;        // debug aid (wg_logical): order in which the logical workgroups are dispatched
};

// Logical workgroup of hardware workgroup `bid` of `n`: as launched (order 0), reversed (1), or
// rotated by half the grid (2).  The result of a launch must not depend on the order; a test
// checks that it is bitwise the same.
__device__ __forceinline__ int wg_logical(int bid, int n, int order) {
    if (order == 1) return n - 1 - bid;
    if (order == 2) return (bid + n / 2) % n;
    return bid;
}

// The LSE merge of two results over disjoint key sets, (O_c, lse_c) and (O_r, lse_r), in the
// natural-log domain: returns the merged LSE and sets the weights, O = wc O_c + wr O_r.  A part
// with LSE -inf (no keys) has weight 0, so merging with it is the identity; both -inf give
// LSE -inf and weights 0 (O = 0); a NaN in either gives NaN weights and LSE.
__device__ __forceinline__ float fold_weights(float lse_c, float lse_r, float& wc, float& wr) {
    if (lse_c != lse_c || lse_r != lse_r) {
        wc = wr = __builtin_nanf("");
        return __builtin_nanf("");
    }
    const float m = fmaxf(lse_c, lse_r);
    if (m == -INFINITY) {
        wc = wr = 0.f;
        return -INFINITY;
    }
    const float ec = expf(lse_c - m), er = expf(lse_r - m), s = ec + er;
    wc = ec / s;
    wr = er / s;
    return m + logf(s);
}

// Query rows per query tile of the bf16 kernel, and the first unit of stream-K run w.
constexpr int kSkRows = 256;
__host__ __device__ inline int64_t sk_start(int64_t U, int w, int n_wgs) { return U * w / n_wgs; }

// Partial slot of a tail segment.  A run's first segment (seg 0) takes slot w; a second segment
// (seg 1) starts at the first unit of tail tile j >= 1, continuing the run from tile j - 1, and
// takes slot n_runs + j - 1.  Runs are at most T units long, so at most one run crosses each
// tile boundary: the slots are distinct and number fewer than n_runs + n_tail.
__host__ __device__ inline int sk_slot(int w, int seg, int j, int n_runs) { return seg == 0 ? w : n_runs + j - 1; }

// The work queues of a persistent launch: 16 counters, each in its own 256-byte line.  Counter
// x < 8 hands out the whole query tiles of XCD x, counter 8 + x its tail runs.
constexpr int kWorkQueueStride = 64;
constexpr int kWorkQueueWords = 16 * kWorkQueueStride;

// The next item of a persistent workgroup on XCD xcd (FwdArgs::persist: a grid of G
// workgroups took items 0 .. G-1 first).  The remaining items are split by b % 8 == x, the XCD
// a round-robin dispatch would give them (so xcd_remap's locality holds), over 8 queues of whole
// query tiles (counter x: items G <= b < n_whole) and 8 queues of tail runs (counter 8 + x:
// items max(G, n_whole) <= b < n_items), each handed out in increasing order.  The workgroup takes
// from its own XCD's whole-tile queue, then from the others' (the longest items go first), then
// from the tail queues in the same order; -1 when all are empty.  A queue found empty is marked
// in `empty` and not asked again.  Relaxed atomics: an item only needs a unique index, and
// items write disjoint outputs.
__device__ __forceinline__ int wq_next(unsigned* wq, int xcd, int G, int n_whole, int n_items, unsigned& empty) {
#pragma unroll 1
    for (int k = 0; k < 16; ++k) {
        const int x = (xcd + k) & 7, qi = (k & 8) | x;
        const int lo = k < 8 ? G : (G > n_whole ? G : n_whole), hi = k < 8 ? n_whole : n_items;
        const int first = lo + ((x - lo) & 7);  // the queue's first item
        if ((empty >> qi) & 1u) continue;
        if (first < hi) {
            const int b = first + 8 * (int)atomicAdd(wq + qi * kWorkQueueStride, 1u);
            if (b < hi) return b;
        }
        empty |= 1u << qi;
    }
    return -1;
}

// Merge of the stream-K partials of query tiles n_dp .. n_q-1 (see FwdArgs).
struct SkFixupArgs {
    int B, H, Sq, D;
    int n_qt;            // query tiles per (b, h): ceil(Sq / kSkRows)
    int T;               // key tiles per query tile
    int n_dp, n_q, sk_wgs;
    int sk_parts;        // as in FwdArgs
    const float* sk_o;
    const float* sk_lse;
    void* o;             // final output, strides os, bf16 or fp32
    Strides os;
    int o_bf16;
    float* lse;          // [B, H, Sq]
    const float* run_o;  // running result folded in as one more part (see FwdArgs), or null
    const float* run_lse;
};

// Merge of up to kMaxMergeParts fp32 partials (contiguous [B,H,Sq,D] / [B,H,Sq]).
constexpr int kMaxMergeParts = 64;
struct MergeArgs {
    int n;
    const float* o_parts[kMaxMergeParts];
    const float* lse_parts[kMaxMergeParts];
    int B, H, Sq, D;
    void* o;
    Strides os;
    int o_bf16;
    float* lse;
};

// Ulysses re-layout between a strided [B, H, S, D] tensor (strides st, unit d stride) and the
// packed [n][S][B][Hg][D] buffer (Hg = H / n) whose part j goes to, or came from, rank j.
struct RelayoutArgs {
    const void* src;
    void* dst;
    Strides st;          // of the strided side (elements)
    int n, B, S, Hg, D;  // H = n * Hg
    int esize;           // bytes per element (2 or 4)
};

// FP8 (OCP E4M3) attention over one chunk of keys, D = 128.  q, k, v hold E4M3 codes (one
// byte per element; strides in elements, i.e. bytes); their values are the codes times
// per-tensor descales.  vt: V^T tiles written by launch_fp8_pack_v, kFp8TileBytes per
// (b, h, 64-key tile), tile-major per head.
constexpr int kFp8TileBytes = 8192;
struct Fp8Args {
    const void* q;
    const void* k;
    const void* v;
    Strides qs, ks, vs;
    void* vt;
    void* o;             // [B, H, Sq, 128], o_bf16 ? bf16 : fp32, strides os
    Strides os;
    int o_bf16;
    float* lse;          // [B, H, Sq] fp32 contiguous, natural log
    int B, H, Sq, Skv;   // Skv >= 1
    float c;             // scale * log2(e) * q_descale * k_descale
    float v_descale;
    // Balanced tail and dispatch, as in FwdArgs (query tiles of kSkRows rows,
    // T = fp8_key_tiles(Skv))
    int n_dp;
    int sk_wgs;          // runs of the tail; 0 = no tail
    int sk_parts;
    float* sk_o;
    float* sk_lse;
    int persist;
    unsigned* wq;
    int wg_order;        // as in FwdArgs
};
int fp8_key_tiles(int Skv);

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_sk_fixup(const SkFixupArgs& a, hipStream_t stream);
// Zeroes the kWorkQueueWords-word work queues of a persistent launch (a kernel, not a memset).
hipError_t launch_wq_clear(unsigned* wq, hipStream_t stream);
hipError_t launch_fp8_pack_v(const Fp8Args& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);
// O = 0 and LSE = -inf for every row (a chunk without keys).
// pack: src strided -> dst packed; unpack: src packed -> dst strided.
hipError_t launch_ulysses_relayout(const RelayoutArgs& a, bool pack, hipStream_t stream);
hipError_t launch_fill_empty(void* o, Strides os, int o_bf16, float* lse, int B, int H, int Sq, int D,
                             hipStream_t stream);

}  // namespace lsdit
