// C ABI of libattn.so: argument checking, dispatch to the HIP kernels, and
// the shard driver that runs the key/value chunk loop on one GPU.
//
// The chunk loop is the per-rank work of Ring Attention and AllGather-KV
// context parallelism (NVIDIA Technical Blog "Scaling AI Inference Across
// Multiple GPUs Using NVIDIA TensorRT with Multi-Device Inference Support",
// sections "Ring Attention" and "AllGather KV"): the chunks of keys are folded
// into the output one after another by an online softmax.  Three schedules are
// offered: one kernel that walks every chunk in order with the softmax state in
// registers (fused), or one kernel per chunk with the partial outputs merged by
// their log-sum-exp weights, either pairwise after every chunk as a ring does
// (online) or all at the end (n-way).  All give attention over the whole key
// sequence.
#include "attn.h"

#include <math.h>
#include <string.h>

#include "kernels.h"

namespace {

using lsdit::FwdArgs;
using lsdit::MergeArgs;
using lsdit::Strides;

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t esize(attn_dtype_t d) { return d == ATTN_BF16 ? 2 : 4; }
inline bool valid_dtype(attn_dtype_t d) { return d == ATTN_F32 || d == ATTN_BF16; }
inline Strides S(attn_strides_t s) { return Strides{s.b, s.h, s.s}; }
inline Strides contiguous(int H, int Sq, int D) {
    return Strides{(int64_t)H * Sq * D, (int64_t)Sq * D, (int64_t)D};
}

bool strides_ok(attn_strides_t s, size_t es) {
    if (s.b < 0 || s.h < 0 || s.s < 0) return false;
    return (s.b * (int64_t)es) % 16 == 0 && (s.h * (int64_t)es) % 16 == 0 && (s.s * (int64_t)es) % 16 == 0;
}

// Checks shared by attn_chunk_fwd and attn_shard_fwd (Skv < 0 means "not applicable").
attn_status_t check_common(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks, const void* v,
                           attn_strides_t vs, attn_dtype_t in_dt, int32_t B, int32_t H, int32_t Sq, int32_t Skv,
                           int32_t D, float scale, const void* o, attn_strides_t os, attn_dtype_t o_dt,
                           const float* lse, bool* noop) {
    *noop = false;
    if (!valid_dtype(in_dt) || !valid_dtype(o_dt)) return ATTN_ERR_DTYPE;
    if (in_dt == ATTN_F32 && o_dt != ATTN_F32) return ATTN_ERR_DTYPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || Sq < 0) return ATTN_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return ATTN_ERR_SHAPE;
    if ((int64_t)B * H * Sq == 0) {
        *noop = true;
        return ATTN_OK;
    }
    if (!q || !o || !lse) return ATTN_ERR_NULL;
    if (Skv != 0 && (!k || !v)) return ATTN_ERR_NULL;
    const size_t ie = esize(in_dt), oe = esize(o_dt);
    if (!aligned16(q) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
    if (!strides_ok(qs, ie) || !strides_ok(os, oe)) return ATTN_ERR_ALIGN;
    if (Skv != 0) {
        if (!aligned16(k) || !aligned16(v)) return ATTN_ERR_ALIGN;
        if (!strides_ok(ks, ie) || !strides_ok(vs, ie)) return ATTN_ERR_ALIGN;
        // the bf16 kernel addresses one head's K/V rows with 32-bit byte offsets
        const int64_t lim = (int64_t)1 << 31;
        if (in_dt == ATTN_BF16 && ((int64_t)(Skv + 256) * ks.s * 2 >= lim || (int64_t)(Skv + 256) * vs.s * 2 >= lim))
            return ATTN_ERR_UNSUPPORTED;
    }
    return ATTN_OK;
}

// One launch over a.n_chunks >= 1 non-empty chunks.
hipError_t run_fwd(const FwdArgs& a, attn_dtype_t in_dt, hipStream_t st) {
    return in_dt == ATTN_BF16 ? lsdit::launch_fwd_bf16(a, st) : lsdit::launch_fwd_f32(a, st);
}

size_t slot_bytes(int32_t B, int32_t H, int32_t Sq, int32_t D) {
    const size_t rows = (size_t)B * H * Sq;
    return align_up(rows * D * 4) + align_up(rows * 4);
}

int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

// The balanced tail of the bf16 kernel (FwdArgs): when its n_q query tiles leave CUs idle in
// the last round, the full rounds run whole query tiles and the last round's work is spread
// evenly over the CUs as runs of (query tile, key tile) units, whose partials the fix-up kernel
// merges.  Worth it when the idle part of the last round is at least kSkMinSaving key tiles
// per CU: the runs' pipeline fill and drain, their partials and the fix-up launch cost about
// as much as 20-30 key tiles (at 22 tiles, the 4,608-token image shape ran 4.5% slower with the
// tail; at 200-430 tiles the 44,160-key Ulysses and ring shares ran 2.7-2.8% faster).
struct SkPlan {
    int n_dp = 0;    // query tiles run whole
    int sk_wgs = 0;  // workgroups of the tail (0 = no tail)
};
constexpr int64_t kSkMinSaving = 64;

SkPlan sk_plan(int64_t n_q, int64_t T, int cus) {
    SkPlan p;
    if (n_q <= 0 || T <= 0 || cus <= 0 || n_q > 0x7FFFFFFF) return p;
    const int64_t rem = n_q % cus;
    if (rem == 0 || T * (cus - rem) / cus < kSkMinSaving) return p;
    const int64_t U = rem * T;  // > rem, since T >= kSkMinSaving: every run is at most T long
    p.n_dp = (int)(n_q - rem);
    p.sk_wgs = (int)(U < cus ? U : cus);
    return p;
}

// Query tiles of the bf16 kernel, and the workspace of its tail: 2 slots per workgroup.
int64_t n_qtiles(int64_t B, int64_t H, int64_t Sq) { return B * H * ((Sq + lsdit::kSkRows - 1) / lsdit::kSkRows); }
size_t sk_o_bytes(int sk_wgs, int D) { return align_up((size_t)2 * sk_wgs * lsdit::kSkRows * D * 4); }
size_t sk_bytes(int sk_wgs, int D) { return sk_o_bytes(sk_wgs, D) + align_up((size_t)2 * sk_wgs * lsdit::kSkRows * 4); }

// The FP8 call's workspace: V^T tiles, then the balanced tail's partials when it runs.
size_t fp8_vt_bytes(int64_t B, int64_t H, int32_t Skv) {
    return (size_t)B * H * lsdit::fp8_key_tiles(Skv) * lsdit::kFp8TileBytes;
}
SkPlan fp8_plan(int64_t B, int64_t H, int64_t Sq, int32_t Skv) {
    return sk_plan(n_qtiles(B, H, Sq), lsdit::fp8_key_tiles(Skv), device_cus());
}

int slots_for(uint32_t flags, int32_t n) {
    if (n <= 1) return 0;
    if (flags == ATTN_MERGE_NWAY) return n;
    if (flags == ATTN_MERGE_ONLINE) return 2;
    if (flags == ATTN_MERGE_FUSED) return 0;  // one kernel, no partials
    return -1;
}

}  // namespace

extern "C" {

attn_status_t attn_chunk_fwd(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks, const void* v,
                             attn_strides_t vs, attn_dtype_t in_dt, int32_t B, int32_t H, int32_t Sq, int32_t Skv,
                             int32_t D, float scale, void* o, attn_strides_t os, attn_dtype_t o_dt, float* lse,
                             attn_stream_t stream) {
    if (Skv < 0) return ATTN_ERR_SHAPE;
    bool noop = false;
    attn_status_t st = check_common(q, qs, k, ks, v, vs, in_dt, B, H, Sq, Skv, D, scale, o, os, o_dt, lse, &noop);
    if (st != ATTN_OK || noop) return st;
    const hipStream_t s = (hipStream_t)stream;
    if (Skv == 0)  // no keys: O = 0, LSE = -inf
        return lsdit::launch_fill_empty(o, S(os), o_dt == ATTN_BF16, lse, B, H, Sq, D, s) == hipSuccess
                   ? ATTN_OK
                   : ATTN_ERR_HIP;
    FwdArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.qs = S(qs); a.ks = S(ks); a.vs = S(vs);
    a.o = o; a.os = S(os); a.o_bf16 = o_dt == ATTN_BF16;
    a.lse = lse;
    a.B = B; a.H = H; a.Sq = Sq; a.Skv = Skv; a.D = D;
    a.scale = scale;
    a.n_chunks = 1;
    a.chunk_row[0] = 0;
    a.chunk_len[0] = Skv;
    return run_fwd(a, in_dt, s) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_lse_merge(int32_t n, const float* const* o_parts, const float* const* lse_parts, int32_t B,
                             int32_t H, int32_t Sq, int32_t D, void* o_out, attn_strides_t os, attn_dtype_t o_dt,
                             float* lse_out, attn_stream_t stream) {
    if (!valid_dtype(o_dt)) return ATTN_ERR_DTYPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (n < 1 || B < 0 || H < 0 || Sq < 0) return ATTN_ERR_SHAPE;
    if (n > ATTN_MAX_CHUNKS || n > lsdit::kMaxMergeParts) return ATTN_ERR_UNSUPPORTED;
    if ((int64_t)B * H * Sq == 0) return ATTN_OK;
    if (!o_parts || !lse_parts || !o_out || !lse_out) return ATTN_ERR_NULL;
    MergeArgs m{};
    for (int c = 0; c < n; ++c) {
        if (!o_parts[c] || !lse_parts[c]) return ATTN_ERR_NULL;
        if (!aligned16(o_parts[c]) || !aligned16(lse_parts[c])) return ATTN_ERR_ALIGN;
        m.o_parts[c] = o_parts[c];
        m.lse_parts[c] = lse_parts[c];
    }
    if (!aligned16(o_out) || !aligned16(lse_out) || !strides_ok(os, esize(o_dt))) return ATTN_ERR_ALIGN;
    m.n = n;
    m.B = B; m.H = H; m.Sq = Sq; m.D = D;
    m.o = o_out; m.os = S(os); m.o_bf16 = o_dt == ATTN_BF16; m.lse = lse_out;
    return lsdit::launch_lse_merge(m, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_shard_workspace_size(int32_t B, int32_t H, int32_t Sq, int32_t D, int32_t n_chunks, uint32_t flags) {
    if (B < 0 || H < 0 || Sq < 0 || (D != 64 && D != 128) || n_chunks < 1 || n_chunks > ATTN_MAX_CHUNKS) return 0;
    if (flags == ATTN_MERGE_FUSED || n_chunks == 1) {
        // room for the balanced tail of shapes whose query tiles leave the last round part-full
        // (whether it runs also depends on the key count)
        const int cus = device_cus();
        const int64_t n_q = n_qtiles(B, H, Sq);
        return n_q % cus != 0 ? sk_bytes(cus, D) : 0;
    }
    const int slots = slots_for(flags, n_chunks);
    if (slots <= 0) return 0;
    return (size_t)slots * slot_bytes(B, H, Sq, D);
}

attn_status_t attn_shard_fwd(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks, const void* v,
                             attn_strides_t vs, attn_dtype_t in_dt, int32_t B, int32_t H, int32_t Sq, int32_t D,
                             float scale, int32_t n_chunks, const int32_t* chunk_len, const int32_t* order,
                             uint32_t flags, void* workspace, size_t ws_bytes, void* o, attn_strides_t os,
                             attn_dtype_t o_dt, float* lse, attn_stream_t stream) {
    // ---- chunk plan (host): lengths, offsets, processing order
    if (n_chunks < 1) return ATTN_ERR_SHAPE;
    if (n_chunks > ATTN_MAX_CHUNKS) return ATTN_ERR_UNSUPPORTED;
    if (!chunk_len) return ATTN_ERR_NULL;
    int64_t off[ATTN_MAX_CHUNKS];
    int64_t total = 0;
    for (int c = 0; c < n_chunks; ++c) {
        if (chunk_len[c] < 0) return ATTN_ERR_SHAPE;
        off[c] = total;
        total += chunk_len[c];
    }
    if (total > 0x7FFFFFFF) return ATTN_ERR_SHAPE;
    int32_t ord[ATTN_MAX_CHUNKS];
    bool seen[ATTN_MAX_CHUNKS] = {};
    for (int t = 0; t < n_chunks; ++t) {
        const int32_t c = order ? order[t] : t;
        if (c < 0 || c >= n_chunks || seen[c]) return ATTN_ERR_SHAPE;
        seen[c] = true;
        ord[t] = c;
    }
    if (n_chunks > 1 && slots_for(flags, n_chunks) < 0) return ATTN_ERR_UNSUPPORTED;
    static_assert(ATTN_MAX_CHUNKS <= lsdit::kMaxChunks, "chunk table too small");

    bool noop = false;
    attn_status_t st = check_common(q, qs, k, ks, v, vs, in_dt, B, H, Sq, (int32_t)total, D, scale, o, os, o_dt,
                                    lse, &noop);
    if (st != ATTN_OK || noop) return st;

    // chunks without keys carry no weight: drop them from the schedule
    int32_t live[ATTN_MAX_CHUNKS];
    int n_live = 0;
    for (int t = 0; t < n_chunks; ++t)
        if (chunk_len[ord[t]] > 0) live[n_live++] = ord[t];

    const size_t need = slots_for(flags, n_chunks) > 0 ? attn_shard_workspace_size(B, H, Sq, D, n_chunks, flags) : 0;
    if (n_live > 1 && need > 0) {
        if (!workspace || ws_bytes < need) return ATTN_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return ATTN_ERR_ALIGN;
    }

    const hipStream_t s = (hipStream_t)stream;
    FwdArgs base{};
    base.q = q; base.k = k; base.v = v;
    base.qs = S(qs); base.ks = S(ks); base.vs = S(vs);
    base.B = B; base.H = H; base.Sq = Sq; base.Skv = (int32_t)total; base.D = D; base.scale = scale;
    auto chunk_args = [&](int c) {  // one chunk, by its rows in the k and v tensors
        FwdArgs a = base;
        a.n_chunks = 1;
        a.chunk_row[0] = (int32_t)off[c];
        a.chunk_len[0] = chunk_len[c];
        return a;
    };
    auto to_final = [&](FwdArgs& a) {
        a.o = o; a.os = S(os); a.o_bf16 = o_dt == ATTN_BF16; a.lse = lse;
    };
    const size_t rows = (size_t)B * H * Sq;
    const Strides cs = contiguous(H, Sq, D);
    auto slot_o = [&](int i) { return (float*)((char*)workspace + (size_t)i * slot_bytes(B, H, Sq, D)); };
    auto slot_lse = [&](int i) { return (float*)((char*)slot_o(i) + align_up(rows * D * 4)); };
    auto ok = [](hipError_t e) { return e == hipSuccess; };

    if (n_live == 0) {
        return ok(lsdit::launch_fill_empty(o, S(os), o_dt == ATTN_BF16, lse, B, H, Sq, D, s)) ? ATTN_OK
                                                                                                : ATTN_ERR_HIP;
    }
    if (n_live == 1 || flags == ATTN_MERGE_FUSED) {
        // one kernel walks the chunks in processing order, the online-softmax state in registers
        FwdArgs a = base;
        a.n_chunks = n_live;
        for (int t = 0; t < n_live; ++t) {
            a.chunk_row[t] = (int32_t)off[live[t]];
            a.chunk_len[t] = chunk_len[live[t]];
        }
        to_final(a);
        // query tiles that leave the last round part-full: spread that round's work evenly
        // (the balanced tail), as far as the workspace allows
        const bool ws_ok = workspace && (reinterpret_cast<uintptr_t>(workspace) & 15u) == 0;
        int64_t T = 0;  // key tiles of the chunk list, as the kernel counts them
        for (int t = 0; t < n_live; ++t) T += (chunk_len[live[t]] + 63) / 64;
        const int64_t n_q = n_qtiles(B, H, Sq);
        const SkPlan p = in_dt == ATTN_BF16 ? sk_plan(n_q, T, device_cus()) : SkPlan{};
        if (p.sk_wgs == 0 || !ws_ok || ws_bytes < sk_bytes(p.sk_wgs, D))
            return ok(run_fwd(a, in_dt, s)) ? ATTN_OK : ATTN_ERR_HIP;
        a.n_dp = p.n_dp;
        a.sk_wgs = p.sk_wgs;
        a.sk_o = (float*)workspace;
        a.sk_lse = (float*)((char*)workspace + sk_o_bytes(p.sk_wgs, D));
        if (!ok(run_fwd(a, in_dt, s))) return ATTN_ERR_HIP;
        lsdit::SkFixupArgs f{};
        f.B = B; f.H = H; f.Sq = Sq; f.D = D;
        f.n_qt = (int)((Sq + lsdit::kSkRows - 1) / lsdit::kSkRows);
        f.T = (int)T;
        f.n_dp = p.n_dp; f.n_q = (int)n_q; f.sk_wgs = p.sk_wgs;
        f.sk_o = a.sk_o; f.sk_lse = a.sk_lse;
        f.o = o; f.os = S(os); f.o_bf16 = o_dt == ATTN_BF16; f.lse = lse;
        return ok(lsdit::launch_sk_fixup(f, s)) ? ATTN_OK : ATTN_ERR_HIP;
    }

    MergeArgs m{};
    m.B = B; m.H = H; m.Sq = Sq; m.D = D;
    if (flags == ATTN_MERGE_ONLINE) {
        for (int t = 0; t < n_live; ++t) {
            FwdArgs a = chunk_args(live[t]);
            const int slot = t == 0 ? 0 : 1;
            a.o = slot_o(slot); a.os = cs; a.o_bf16 = 0; a.lse = slot_lse(slot);
            if (!ok(run_fwd(a, in_dt, s))) return ATTN_ERR_HIP;
            if (t == 0) continue;
            m.n = 2;
            m.o_parts[0] = slot_o(0); m.lse_parts[0] = slot_lse(0);
            m.o_parts[1] = slot_o(1); m.lse_parts[1] = slot_lse(1);
            if (t == n_live - 1) {
                m.o = o; m.os = S(os); m.o_bf16 = o_dt == ATTN_BF16; m.lse = lse;
            } else {
                m.o = slot_o(0); m.os = cs; m.o_bf16 = 0; m.lse = slot_lse(0);
            }
            if (!ok(lsdit::launch_lse_merge(m, s))) return ATTN_ERR_HIP;
        }
        return ATTN_OK;
    }

    // ATTN_MERGE_NWAY
    for (int t = 0; t < n_live; ++t) {
        FwdArgs a = chunk_args(live[t]);
        a.o = slot_o(t); a.os = cs; a.o_bf16 = 0; a.lse = slot_lse(t);
        if (!ok(run_fwd(a, in_dt, s))) return ATTN_ERR_HIP;
        m.o_parts[t] = slot_o(t);
        m.lse_parts[t] = slot_lse(t);
    }
    m.n = n_live;
    m.o = o; m.os = S(os); m.o_bf16 = o_dt == ATTN_BF16; m.lse = lse;
    return ok(lsdit::launch_lse_merge(m, s)) ? ATTN_OK : ATTN_ERR_HIP;
}

namespace {

attn_status_t relayout(const void* src, void* dst, attn_strides_t xs, attn_dtype_t dt, int32_t B,
                       int32_t H, int32_t S, int32_t D, int32_t n, bool pack, hipStream_t stream) {
    if (!valid_dtype(dt)) return ATTN_ERR_DTYPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || S < 0 || n < 1 || H % n != 0) return ATTN_ERR_SHAPE;
    if ((int64_t)B * H * S == 0) return ATTN_OK;
    if (!src || !dst) return ATTN_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst) || !strides_ok(xs, esize(dt))) return ATTN_ERR_ALIGN;
    lsdit::RelayoutArgs a{};
    a.src = src; a.dst = dst; a.st = Strides{xs.b, xs.h, xs.s};
    a.n = n; a.B = B; a.S = S; a.Hg = H / n; a.D = D; a.esize = (int)esize(dt);
    return lsdit::launch_ulysses_relayout(a, pack, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

attn_status_t attn_ulysses_pack(const void* x, attn_strides_t xs, attn_dtype_t dt, int32_t B, int32_t H, int32_t S,
                                int32_t D, int32_t n, void* packed, attn_stream_t stream) {
    return relayout(x, packed, xs, dt, B, H, S, D, n, true, (hipStream_t)stream);
}

attn_status_t attn_ulysses_unpack(const void* packed, attn_dtype_t dt, int32_t B, int32_t H, int32_t S, int32_t D,
                                  int32_t n, void* x, attn_strides_t xs, attn_stream_t stream) {
    return relayout(packed, x, xs, dt, B, H, S, D, n, false, (hipStream_t)stream);
}

size_t attn_fp8_workspace_size(int32_t B, int32_t H, int32_t Sq, int32_t Skv, int32_t D) {
    if (B <= 0 || H <= 0 || Sq < 0 || Skv <= 0 || D != 128) return 0;
    const SkPlan p = fp8_plan(B, H, Sq, Skv);
    return fp8_vt_bytes(B, H, Skv) + (p.sk_wgs ? sk_bytes(p.sk_wgs, D) : 0);
}

attn_status_t attn_chunk_fwd_fp8(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks, const void* v,
                                 attn_strides_t vs, float q_descale, float k_descale, float v_descale, int32_t B,
                                 int32_t H, int32_t Sq, int32_t Skv, int32_t D, float scale, void* workspace,
                                 size_t ws_bytes, void* o, attn_strides_t os, attn_dtype_t o_dt, float* lse,
                                 attn_stream_t stream) {
    if (!valid_dtype(o_dt)) return ATTN_ERR_DTYPE;
    if (D != 128) return ATTN_ERR_UNSUPPORTED;
    if (B < 0 || H < 0 || Sq < 0 || Skv < 0) return ATTN_ERR_SHAPE;
    for (float x : {scale, q_descale, k_descale, v_descale})
        if (!(x > 0.f) || !isfinite(x)) return ATTN_ERR_SHAPE;
    if ((int64_t)B * H * Sq == 0) return ATTN_OK;
    if (!q || !o || !lse) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
    if (!strides_ok(qs, 1) || !strides_ok(os, esize(o_dt))) return ATTN_ERR_ALIGN;
    const hipStream_t s = (hipStream_t)stream;
    if (Skv == 0)
        return lsdit::launch_fill_empty(o, S(os), o_dt == ATTN_BF16, lse, B, H, Sq, D, s) == hipSuccess
                   ? ATTN_OK
                   : ATTN_ERR_HIP;
    if (!k || !v || !workspace) return ATTN_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(workspace)) return ATTN_ERR_ALIGN;
    if (!strides_ok(ks, 1) || !strides_ok(vs, 1)) return ATTN_ERR_ALIGN;
    // 32-bit buffer offsets: one head's K rows and V^T tiles, plus the four tiles the kernel
    // fetches past the end
    if ((int64_t)(Skv + 320) * ks.s >= ((int64_t)1 << 31) || Skv >= (1 << 23)) return ATTN_ERR_UNSUPPORTED;
    if (ws_bytes < attn_fp8_workspace_size(B, H, Sq, Skv, D)) return ATTN_ERR_WORKSPACE;
    lsdit::Fp8Args a{};
    a.q = q; a.k = k; a.v = v;
    a.qs = S(qs); a.ks = S(ks); a.vs = S(vs);
    a.vt = workspace;
    a.o = o; a.os = S(os); a.o_bf16 = o_dt == ATTN_BF16;
    a.lse = lse;
    a.B = B; a.H = H; a.Sq = Sq; a.Skv = Skv;
    a.c = (float)((double)scale * 1.4426950408889634 * (double)q_descale * (double)k_descale);
    a.v_descale = v_descale;
    if (!(a.c > 0.f) || !isfinite(a.c)) return ATTN_ERR_SHAPE;
    // the balanced tail, as in attn_shard_fwd, its partials after V^T in the workspace
    const SkPlan p = fp8_plan(B, H, Sq, Skv);
    if (p.sk_wgs) {
        a.n_dp = p.n_dp;
        a.sk_wgs = p.sk_wgs;
        a.sk_o = (float*)((char*)workspace + fp8_vt_bytes(B, H, Skv));
        a.sk_lse = (float*)((char*)a.sk_o + sk_o_bytes(p.sk_wgs, D));
    }
    if (lsdit::launch_fp8_pack_v(a, s) != hipSuccess) return ATTN_ERR_HIP;
    if (lsdit::launch_fwd_fp8(a, s) != hipSuccess) return ATTN_ERR_HIP;
    if (!p.sk_wgs) return ATTN_OK;
    lsdit::SkFixupArgs f{};
    f.B = B; f.H = H; f.Sq = Sq; f.D = D;
    f.n_qt = (int)((Sq + lsdit::kSkRows - 1) / lsdit::kSkRows);
    f.T = lsdit::fp8_key_tiles(Skv);
    f.n_dp = p.n_dp; f.n_q = (int)n_qtiles(B, H, Sq); f.sk_wgs = p.sk_wgs;
    f.sk_o = a.sk_o; f.sk_lse = a.sk_lse;
    f.o = o; f.os = S(os); f.o_bf16 = o_dt == ATTN_BF16; f.lse = lse;
    return lsdit::launch_sk_fixup(f, s) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

const char* attn_status_str(attn_status_t s) {
    switch (s) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "invalid shape, scale, chunk lengths or order";
        case ATTN_ERR_DTYPE: return "unsupported dtype combination";
        case ATTN_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
        case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension, chunk count or merge mode";
        case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case ATTN_ERR_HIP: return "HIP kernel launch failed";
    }
    return "unknown status";
}

int32_t attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
