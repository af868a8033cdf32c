// Internal interface between the C-ABI host code (attn_api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
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
    // Balanced tail (bf16 path): sk_wgs > 0 launches n_dp + sk_wgs
    // workgroups.  Workgroups below n_dp take one whole query tile each (query tiles
    // 0 .. n_dp-1 of the n_q = B*H*ceil(Sq/kSkRows) in (b, h, tile) order) and write the final
    // output.  The other query tiles make U = (n_q - n_dp) * T units (query tile, key tile), T
    // key tiles per query tile; stream-K workgroup w takes units [sk_start(U, w, sk_wgs),
    // sk_start(U, w + 1, sk_wgs)): at most two query-tile segments, because sk_wgs > n_q - n_dp
    // makes every range at most T long.  With sk_wgs == 0 the grid is one workgroup per query
    // tile.  Segment i of workgroup w is written as an fp32 partial
    // (normalised by its own row sum) with its natural-log LSE into slot 2w + i: row r of the
    // query tile at sk_o + slot*kSkRows*D + r*D and sk_lse + slot*kSkRows + r.
    // launch_sk_fixup then merges the partials into the final output.
    int n_dp;
    int sk_wgs;          // 0 = no stream-K tail
    float* sk_o;
    float* sk_lse;
};

// Query rows per query tile of the bf16 kernel, and the first unit of stream-K workgroup w.
constexpr int kSkRows = 256;
__host__ __device__ inline int64_t sk_start(int64_t U, int w, int n_wgs) { return U * w / n_wgs; }

// Merge of the stream-K partials of query tiles n_dp .. n_q-1 (see FwdArgs).
struct SkFixupArgs {
    int B, H, Sq, D;
    int n_qt;            // query tiles per (b, h): ceil(Sq / kSkRows)
    int T;               // key tiles per query tile
    int n_dp, n_q, sk_wgs;
    const float* sk_o;
    const float* sk_lse;
    void* o;             // final output, strides os, bf16 or fp32
    Strides os;
    int o_bf16;
    float* lse;          // [B, H, Sq]
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
    // Balanced tail, as in FwdArgs (query tiles of kSkRows rows, T = fp8_key_tiles(Skv))
    int n_dp;
    int sk_wgs;          // 0 = no stream-K tail
    float* sk_o;
    float* sk_lse;
};
int fp8_key_tiles(int Skv);

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_sk_fixup(const SkFixupArgs& a, hipStream_t stream);
hipError_t launch_fp8_pack_v(const Fp8Args& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);
// O = 0 and LSE = -inf for every row (a chunk without keys).
// pack: src strided -> dst packed; unpack: src packed -> dst strided.
hipError_t launch_ulysses_relayout(const RelayoutArgs& a, bool pack, hipStream_t stream);
hipError_t launch_fill_empty(void* o, Strides os, int o_bf16, float* lse, int B, int H, int Sq, int D,
                             hipStream_t stream);

}  // namespace lsdit
