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

// One chunk-attention launch.  Pointers are device pointers.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    Strides qs, ks, vs;
    void* o;             // [B, H, Sq, D], o_bf16 ? bf16 : fp32, strides os
    Strides os;
    int o_bf16;
    float* lse;          // [B, H, Sq] fp32 contiguous
    const float* prev_o; // optional running fp32 result merged in the epilogue (may alias o)
    Strides ps;
    const float* prev_lse;  // [B, H, Sq] (may alias lse); NULL when prev_o is NULL
    int B, H, Sq, Skv, D;
    float scale;
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

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t stream);
// O = 0 and LSE = -inf for every row (a chunk without keys).
hipError_t launch_fill_empty(void* o, Strides os, int o_bf16, float* lse, int B, int H, int Sq, int D,
                             hipStream_t stream);

}  // namespace lsdit
