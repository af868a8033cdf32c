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
    // Split over the keys (bf16 path): n_split > 1 launches n_split workgroups per query
    // tile; split s takes tiles [s*T/n_split, (s+1)*T/n_split) of the T key tiles and writes
    // an fp32 partial (normalised by its own row sum) and its LSE at o + s*split_o_stride and
    // lse + s*split_lse_stride (elements); the partials are then merged by their LSE.
    int n_split;         // 1 = no split
    int64_t split_o_stride, split_lse_stride;
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
};
int fp8_key_tiles(int Skv);

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_fp8_pack_v(const Fp8Args& a, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);
// O = 0 and LSE = -inf for every row (a chunk without keys).
// pack: src strided -> dst packed; unpack: src packed -> dst strided.
hipError_t launch_ulysses_relayout(const RelayoutArgs& a, bool pack, hipStream_t stream);
hipError_t launch_fill_empty(void* o, Strides os, int o_bf16, float* lse, int B, int H, int Sq, int D,
                             hipStream_t stream);

}  // namespace lsdit
