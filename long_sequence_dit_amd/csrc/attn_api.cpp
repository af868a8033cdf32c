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
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

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

// Debug aid: LSDIT_DEBUG_WG_ORDER=reverse (or rotate) dispatches the forward kernels' logical
// workgroups in reversed (or half-rotated) order, so that a test can check that results do not
// depend on which workgroups run together or first.
int debug_wg_order() {
    const char* e = getenv("LSDIT_DEBUG_WG_ORDER");
    if (!e) return 0;
    if (strcmp(e, "reverse") == 0) return 1;
    if (strcmp(e, "rotate") == 0) return 2;
    return 0;
}

// Debug aids for tests: LSDIT_DEBUG_PERSIST=0 never runs a launch persistent, =1 does so for
// every launch of more than one round (whatever its work per CU); LSDIT_DEBUG_TAIL fixes a
// persistent launch's tail: "ranges" for one run of equal units per CU (as a launch of one
// workgroup per item has), an integer r >= 2 for r parts per tail tile.  -1: not set.
int debug_persist() {
    const char* e = getenv("LSDIT_DEBUG_PERSIST");
    if (!e) return -1;
    if (strcmp(e, "0") == 0) return 0;
    if (strcmp(e, "1") == 0) return 1;
    return -1;
}
int debug_tail() {
    const char* e = getenv("LSDIT_DEBUG_TAIL");
    if (!e) return -1;
    if (strcmp(e, "ranges") == 0) return 0;
    const int r = atoi(e);
    return r >= 2 ? r : -1;
}

int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

// The balanced tail (FwdArgs): when a launch's n_q query tiles leave CUs idle in the last round,
// the full rounds run whole query tiles and the last round's work is spread over the CUs as runs
// of (query tile, key tile) units, whose partials the fix-up kernel merges.  Worth it when the
// idle part of the last round is at least min_saving key tiles per CU: the runs' pipeline fill
// and drain, their partials and the fix-up launch cost about as much as 20-30 key tiles (bf16:
// at 22 tiles, the 4,608-token image shape ran 4.5% slower with the tail; at 200-430 tiles the
// 44,160-key Ulysses and ring shares ran 2.7-2.8% faster).  The FP8 kernel's tiles take half the
// time, so its fixed costs weigh about twice as many tiles.
//  * A launch of one workgroup per item cuts the tail into one run of equal units per CU: the
//    hardware deals the runs out as CUs come free, and equal runs end together.
//  * A persistent launch (FwdArgs::persist) cuts every tail tile into r equal parts instead, so
//    that its queues balance the end to a fraction of a query tile.  Parts, unlike runs of equal
//    units, never cross a tile boundary, and the queues hand them out part-major, so that an
//    XCD's runs at one time read the same key range.  r is at most what parts of min_run key
//    tiles and kSkMaxRunsPerCu runs per CU allow: a run's fixed costs (prologue, epilogue, fp32
//    partial, the queue) come to about 9 us, and at 65 key tiles per run they outweighed the
//    balance gained on a box whose XCDs were close.  Among those r it takes the one whose
//    n = r * n_tail parts fill the CUs' last round of parts best (the least ceil(n/cus) /
//    (n/cus) - 1; a larger r unless a smaller one is better by 0.02): the tail's parts all start
//    at about the same time, so a last round that is part-full costs nearly a whole part (the
//    ring share: 1.65 ms at 5 parts, 1.70 at 4 and 1.79-1.81 at 3, whose 288 parts leave 224
//    CUs a second round).  Above 0.3, and with fewer parts than CUs, one run of equal units
//    per CU balances better.
// The persistent launch itself pays off from about kPersistMinTiles key tiles per CU (its
// queues cost a few microseconds per item): the XCDs' clocks differ by up to ~8%, and a static
// grid ends with the slowest XCD (44,160-key shares: 4-7% faster on the slowest boxes, 1% on the
// fastest; the 4,608-token image shape, 121 tiles per CU, ran 3-10% slower persistent).
struct SkPlan {
    int n_dp = 0;    // query tiles run whole
    int sk_wgs = 0;  // runs of the tail (0 = no tail)
    int parts = 0;   // 0: runs of equal units; r >= 2: r parts per tail tile
};
constexpr int64_t kSkMinSavingBf16 = 40;
constexpr int64_t kSkMinSavingFp8 = 64;
constexpr int kSkMaxRunsPerCu = 4;
constexpr int64_t kSkMinRunTiles = 128;
constexpr int64_t kPersistMinTiles = 512;

// persist: the launch is persistent; min_run: the fewest key tiles per part
SkPlan sk_plan(int64_t n_q, int64_t T, int cus, int64_t min_saving, bool persist = false,
               int64_t min_run = kSkMinRunTiles) {
    SkPlan p;
    if (n_q <= 0 || T <= 0 || cus <= 0 || n_q > 0x7FFFFFFF) return p;
    const int64_t rem = n_q % cus;
    if (rem == 0 || T * (cus - rem) / cus < min_saving) return p;
    const int64_t U = rem * T;  // > rem, since T > min_saving >= 1: every run is at most T long
    p.n_dp = (int)(n_q - rem);
    p.sk_wgs = (int)(U < cus ? U : cus);
    if (persist) {
        const int64_t most = ((int64_t)kSkMaxRunsPerCu * cus + rem - 1) / rem;
        const int64_t r_max = T / min_run < most ? T / min_run : most;
        int64_t r = 0;
        double best = 0.3;  // the most a last round of parts may leave idle, relative
        for (int64_t c = r_max; c >= 2; --c) {
            const double per = (double)(c * rem) / cus;
            if (per < 1.0) break;  // fewer parts than CUs
            const double idle = (double)((c * rem + cus - 1) / cus) / per - 1.0;
            if (r == 0 ? idle <= best : idle < best - 0.02) {
                r = c;
                best = idle;
            }
        }
        const int dt = debug_tail();
        if (dt >= 0) r = dt;
        if (r >= 2 && r <= T) {
            p.parts = (int)r;
            p.sk_wgs = (int)(r * rem);
        }
    }
    return p;
}

// Query tiles of the bf16 kernel, and the workspace of its tail: one partial slot per run, and
// for runs of equal units one per tail tile boundary (lsdit::sk_slot), each of kSkRows rows of D
// fp32 values and an LSE.
int64_t n_qtiles(int64_t B, int64_t H, int64_t Sq) { return B * H * ((Sq + lsdit::kSkRows - 1) / lsdit::kSkRows); }
int64_t sk_slots(const SkPlan& p, int64_t n_q) {
    return p.sk_wgs == 0 ? 0 : p.parts ? p.sk_wgs : p.sk_wgs + (n_q - p.n_dp);
}
size_t sk_o_bytes(int64_t n_slots, int D) { return align_up((size_t)n_slots * lsdit::kSkRows * D * 4); }
size_t sk_bytes(int64_t n_slots, int D) { return sk_o_bytes(n_slots, D) + align_up((size_t)n_slots * lsdit::kSkRows * 4); }
// The work queues of a persistent launch, in the workspace before the tail's partials: present
// when the query tiles take more than one round.
constexpr size_t kWqBytes = (size_t)lsdit::kWorkQueueWords * 4;
size_t wq_bytes(int64_t n_q, int cus) { return n_q > cus ? kWqBytes : 0; }
// The most room a shape's tail can take: up to kSkMaxRunsPerCu runs per CU (rounded up to whole
// parts per tail tile) when persistent
size_t tail_room(int64_t n_q, int cus, int D) {
    const int64_t rem = n_q % cus;
    if (rem == 0) return 0;
    return sk_bytes((n_q > cus ? kSkMaxRunsPerCu : 1) * (int64_t)cus + rem, D);
}

// The persistent launch and its tail for a launch of n_q query tiles against T key tiles: bf16
// (weight 1) or FP8, whose tiles take about half the time (weight 2: twice the tiles per CU
// before the queues pay, 1.5 times the key tiles per part).  persist_ok: the caller has room for
// the work queues.
struct LaunchPlan {
    bool persist = false;
    SkPlan sk;
};
LaunchPlan launch_plan(int64_t n_q, int64_t T, int cus, int64_t min_saving, int64_t weight, bool persist_ok) {
    LaunchPlan lp;
    lp.persist = persist_ok && n_q > cus && n_q * T >= kPersistMinTiles * weight * cus;
    if (debug_persist() >= 0) lp.persist = persist_ok && n_q > cus && debug_persist() == 1;
    // FP8 parts of 256 key tiles ran 0.8% slower than parts of 172-230 at the full sequence
    lp.sk = sk_plan(n_q, T, cus, min_saving, lp.persist, weight == 1 ? kSkMinRunTiles : kSkMinRunTiles * 3 / 2);
    return lp;
}

// The FP8 call's workspace: V^T tiles, then, for a persistent launch, the work queues, then the
// balanced tail's partials when it runs.
size_t fp8_vt_bytes(int64_t B, int64_t H, int32_t Skv) {
    return (size_t)B * H * lsdit::fp8_key_tiles(Skv) * lsdit::kFp8TileBytes;
}
LaunchPlan fp8_plan(int64_t B, int64_t H, int64_t Sq, int32_t Skv) {
    return launch_plan(n_qtiles(B, H, Sq), lsdit::fp8_key_tiles(Skv), device_cus(), kSkMinSavingFp8, 2, true);
}

// fp32 chunk slots of a schedule: NWAY keeps every chunk's partial, ONLINE one running result
// (each chunk's launch folds into it in its epilogue), FUSED none (one kernel, no partials).
int slots_for(uint32_t flags, int32_t n) {
    if (n <= 1) return 0;
    if (flags == ATTN_MERGE_NWAY) return n;
    if (flags == ATTN_MERGE_ONLINE) return 1;
    if (flags == ATTN_MERGE_FUSED) return 0;
    return -1;
}


// ---- the static scratch of attn_shard_fwd_noalloc: the balanced tail's partials (fp32 O, then
// fp32 LSE, as in a workspace) of at most kScratchTailWgs runs at D <= 128 (launches one
// workgroup per item, at most one run per CU: fewer than 2 * kScratchTailWgs slots).
constexpr int kScratchTailWgs = 256;
constexpr size_t kScratchBytes = ((size_t)2 * kScratchTailWgs * lsdit::kSkRows * 128 * 4 + kAlign - 1) / kAlign * kAlign +
                                 ((size_t)2 * kScratchTailWgs * lsdit::kSkRows * 4 + kAlign - 1) / kAlign * kAlign;
static_assert(kScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES, "2 * 256 slots of 256 rows: 128 fp32 values and an LSE each");

}  // namespace

// Every device holds its own copy of this array, from the library's first use on the device
// until the process ends.  In host code `scratch` names a host-side stand-in: its device address
// comes from hipGetSymbolAddress (scratch_address), and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept: the lookup is the set-up, later calls reuse the address.
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static std::atomic<void*> addr[64];
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        static std::mutex mu;
        std::lock_guard<std::mutex> g(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

// The shard driver behind attn_shard_fwd and attn_shard_fwd_noalloc.  With `scratch` set, the
// balanced tail's partials go to the library's static scratch array (workspace and ws_bytes are
// then ignored) and its plan spreads over at most kScratchTailWgs workgroups.
attn_status_t shard_fwd_impl(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks, const void* v,
                             attn_strides_t vs, attn_dtype_t in_dt, int32_t B, int32_t H, int32_t Sq, int32_t D,
                             float scale, int32_t n_chunks, const int32_t* chunk_len, const int32_t* order,
                             uint32_t flags, void* workspace, size_t ws_bytes, bool scratch, void* o,
                             attn_strides_t os, attn_dtype_t o_dt, float* lse, attn_stream_t stream) {
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

    // workspace: the chunk slots of the per-chunk schedules, then the balanced tail's partials
    const int n_slots = slots_for(flags, n_chunks) > 0 ? slots_for(flags, n_chunks) : 0;
    const size_t slots_need = (size_t)n_slots * slot_bytes(B, H, Sq, D);
    const bool ws_aligned = (reinterpret_cast<uintptr_t>(workspace) & 15u) == 0;
    if (n_live > 1 && n_slots > 0) {
        if (!workspace || ws_bytes < slots_need) return ATTN_ERR_WORKSPACE;
        if (!ws_aligned) return ATTN_ERR_ALIGN;
    }
    // after the chunk slots: the work queues (shapes of more than one round), then the tail
    const int64_t n_q = n_qtiles(B, H, Sq);
    const int cus = device_cus();
    const size_t wq_need = wq_bytes(n_q, cus);
    unsigned* wq = nullptr;
    void* tail_ws = nullptr;
    size_t tail_bytes = 0;
    if (!scratch && workspace && ws_aligned && ws_bytes >= slots_need + wq_need) {
        if (wq_need) wq = (unsigned*)((char*)workspace + slots_need);
        tail_ws = (char*)workspace + slots_need + wq_need;
        tail_bytes = ws_bytes - slots_need - wq_need;
        if (tail_bytes == 0) tail_ws = nullptr;
    }

    const hipStream_t s = (hipStream_t)stream;
    FwdArgs base{};
    base.q = q; base.k = k; base.v = v;
    base.qs = S(qs); base.ks = S(ks); base.vs = S(vs);
    base.B = B; base.H = H; base.Sq = Sq; base.Skv = (int32_t)total; base.D = D; base.scale = scale;
    base.wg_order = debug_wg_order();
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
    auto to_slot = [&](FwdArgs& a, int i) {
        a.o = slot_o(i); a.os = cs; a.o_bf16 = 0; a.lse = slot_lse(i);
    };
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    const int tail_cus = scratch && cus > kScratchTailWgs ? kScratchTailWgs : cus;

    // One kernel launch over a's chunk list (T key tiles) into a's output, folding in a's running
    // result if it has one.  A bf16 launch of several rounds with enough work per CU runs
    // persistent when the workspace holds the work queues.  When the query tiles leave the last
    // round of CUs part-full, that round's work is spread evenly (the balanced tail) as far as the
    // tail's room allows, and the fix-up kernel merges the runs' partials (and the running result)
    // into the output.
    auto launch = [&](FwdArgs a, int64_t T) -> attn_status_t {
        const bool bf16 = in_dt == ATTN_BF16;
        const LaunchPlan lp = bf16 ? launch_plan(n_q, T, tail_cus, kSkMinSavingBf16, 1, wq != nullptr) : LaunchPlan{};
        if (lp.persist) {
            a.persist = cus;
            a.wq = wq;
        }
        const SkPlan& p = lp.sk;
        const int64_t n_slots = sk_slots(p, n_q);
        void* tw = tail_ws;
        size_t tb = tail_bytes;
        if (scratch && p.sk_wgs) {
            if (sk_bytes(n_slots, D) > kScratchBytes) return ATTN_ERR_WORKSPACE;  // not with D <= 128
            if (!ok(scratch_address(&tw))) return ATTN_ERR_HIP;
            tb = kScratchBytes;
        }
        if (p.sk_wgs == 0 || !tw || tb < sk_bytes(n_slots, D)) return ok(run_fwd(a, in_dt, s)) ? ATTN_OK : ATTN_ERR_HIP;
        a.n_dp = p.n_dp;
        a.sk_wgs = p.sk_wgs;
        a.sk_parts = p.parts;
        a.sk_o = (float*)tw;
        a.sk_lse = (float*)((char*)tw + sk_o_bytes(n_slots, D));
        if (!ok(run_fwd(a, in_dt, s))) return ATTN_ERR_HIP;
        lsdit::SkFixupArgs f{};
        f.B = B; f.H = H; f.Sq = Sq; f.D = D;
        f.n_qt = (int)((Sq + lsdit::kSkRows - 1) / lsdit::kSkRows);
        f.T = (int)T;
        f.n_dp = p.n_dp; f.n_q = (int)n_q; f.sk_wgs = p.sk_wgs; f.sk_parts = p.parts;
        f.sk_o = a.sk_o; f.sk_lse = a.sk_lse;
        f.o = a.o; f.os = a.os; f.o_bf16 = a.o_bf16; f.lse = a.lse;
        f.run_o = a.run_o; f.run_lse = a.run_lse;
        return ok(lsdit::launch_sk_fixup(f, s)) ? ATTN_OK : ATTN_ERR_HIP;
    };
    auto tiles = [](int64_t len) { return (len + 63) / 64; };  // key tiles, as the kernel counts them

    if (n_live == 0) {
        return ok(lsdit::launch_fill_empty(o, S(os), o_dt == ATTN_BF16, lse, B, H, Sq, D, s)) ? ATTN_OK
                                                                                                : ATTN_ERR_HIP;
    }
    if (n_live == 1 || flags == ATTN_MERGE_FUSED) {
        // one kernel walks the chunks in processing order, the online-softmax state in registers
        FwdArgs a = base;
        a.n_chunks = n_live;
        int64_t T = 0;
        for (int t = 0; t < n_live; ++t) {
            a.chunk_row[t] = (int32_t)off[live[t]];
            a.chunk_len[t] = chunk_len[live[t]];
            T += tiles(chunk_len[live[t]]);
        }
        to_final(a);
        return launch(a, T);
    }

    if (flags == ATTN_MERGE_ONLINE) {
        // as a ring receiving one chunk per step: each chunk's launch folds its result into the
        // running fp32 result in slot 0 (in place; the last one into the final output) in its
        // epilogue, by the LSE rule
        for (int t = 0; t < n_live; ++t) {
            FwdArgs a = chunk_args(live[t]);
            if (t > 0) {
                a.run_o = slot_o(0);
                a.run_lse = slot_lse(0);
            }
            if (t == n_live - 1) to_final(a);
            else to_slot(a, 0);
            const attn_status_t st = launch(a, tiles(chunk_len[live[t]]));
            if (st != ATTN_OK) return st;
        }
        return ATTN_OK;
    }

    // ATTN_MERGE_NWAY: every chunk's fp32 partial in its own slot, then one n-way merge
    MergeArgs m{};
    m.B = B; m.H = H; m.Sq = Sq; m.D = D;
    for (int t = 0; t < n_live; ++t) {
        FwdArgs a = chunk_args(live[t]);
        to_slot(a, t);
        const attn_status_t st = launch(a, tiles(chunk_len[live[t]]));
        if (st != ATTN_OK) return st;
        m.o_parts[t] = slot_o(t);
        m.lse_parts[t] = slot_lse(t);
    }
    m.n = n_live;
    m.o = o; m.os = S(os); m.o_bf16 = o_dt == ATTN_BF16; m.lse = lse;
    return ok(lsdit::launch_lse_merge(m, s)) ? ATTN_OK : ATTN_ERR_HIP;
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
    a.wg_order = debug_wg_order();
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
    const int slots = slots_for(flags, n_chunks);
    if (slots < 0) return 0;
    // the chunk slots, then the work queues of shapes of more than one round, then room for the
    // balanced tail of shapes whose query tiles leave the last round part-full (whether the
    // queues and the tail are used also depends on the key count)
    const int cus = device_cus();
    const int64_t n_q = n_qtiles(B, H, Sq);
    return (size_t)slots * slot_bytes(B, H, Sq, D) + wq_bytes(n_q, cus) + tail_room(n_q, cus, D);
}

attn_status_t attn_shard_fwd(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks, const void* v,
                             attn_strides_t vs, attn_dtype_t in_dt, int32_t B, int32_t H, int32_t Sq, int32_t D,
                             float scale, int32_t n_chunks, const int32_t* chunk_len, const int32_t* order,
                             uint32_t flags, void* workspace, size_t ws_bytes, void* o, attn_strides_t os,
                             attn_dtype_t o_dt, float* lse, attn_stream_t stream) {
    return shard_fwd_impl(q, qs, k, ks, v, vs, in_dt, B, H, Sq, D, scale, n_chunks, chunk_len, order, flags,
                          workspace, ws_bytes, false, o, os, o_dt, lse, stream);
}

attn_status_t attn_shard_fwd_noalloc(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks,
                                     const void* v, attn_strides_t vs, attn_dtype_t in_dt, int32_t B, int32_t H,
                                     int32_t Sq, int32_t D, float scale, int32_t n_chunks, const int32_t* chunk_len,
                                     const int32_t* order, void* o, attn_strides_t os, attn_dtype_t o_dt, float* lse,
                                     attn_stream_t stream) {
    return shard_fwd_impl(q, qs, k, ks, v, vs, in_dt, B, H, Sq, D, scale, n_chunks, chunk_len, order,
                          ATTN_MERGE_FUSED, nullptr, 0, true, o, os, o_dt, lse, stream);
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
    const LaunchPlan lp = fp8_plan(B, H, Sq, Skv);
    return fp8_vt_bytes(B, H, Skv) + (lp.persist ? kWqBytes : 0) +
           (lp.sk.sk_wgs ? sk_bytes(sk_slots(lp.sk, n_qtiles(B, H, Sq)), D) : 0);
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
    a.wg_order = debug_wg_order();
    if (!(a.c > 0.f) || !isfinite(a.c)) return ATTN_ERR_SHAPE;
    // the persistent launch and the balanced tail, as in attn_shard_fwd: the work queues, then the
    // tail's partials, after V^T in the workspace
    const LaunchPlan lp = fp8_plan(B, H, Sq, Skv);
    const SkPlan& p = lp.sk;
    char* after_vt = (char*)workspace + fp8_vt_bytes(B, H, Skv);
    if (lp.persist) {
        a.persist = device_cus();
        a.wq = (unsigned*)after_vt;
        after_vt += kWqBytes;
    }
    if (p.sk_wgs) {
        a.n_dp = p.n_dp;
        a.sk_wgs = p.sk_wgs;
        a.sk_parts = p.parts;
        a.sk_o = (float*)after_vt;
        a.sk_lse = (float*)((char*)a.sk_o + sk_o_bytes(sk_slots(p, n_qtiles(B, H, Sq)), D));
    }
    if (lsdit::launch_fp8_pack_v(a, s) != hipSuccess) return ATTN_ERR_HIP;
    if (lsdit::launch_fwd_fp8(a, s) != hipSuccess) return ATTN_ERR_HIP;
    if (!p.sk_wgs) return ATTN_OK;
    lsdit::SkFixupArgs f{};
    f.B = B; f.H = H; f.Sq = Sq; f.D = D;
    f.n_qt = (int)((Sq + lsdit::kSkRows - 1) / lsdit::kSkRows);
    f.T = lsdit::fp8_key_tiles(Skv);
    f.n_dp = p.n_dp; f.n_q = (int)n_qtiles(B, H, Sq); f.sk_wgs = p.sk_wgs; f.sk_parts = p.parts;
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
        default: break;
    }
    return "unknown status";
}

int32_t attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
