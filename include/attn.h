/*
 * attn.h — C ABI of the long-sequence attention library (libattn.so, gfx950).
 *
 * The operation is bidirectional (non-causal) multi-head softmax attention,
 * evaluated blockwise over chunks of the key/value sequence, with the
 * per-chunk partial results combined by their log-sum-exp.  This is the
 * per-GPU work of context parallelism in the NVIDIA Technical Blog "Scaling
 * AI Inference Across Multiple GPUs Using NVIDIA TensorRT with Multi-Device
 * Inference Support": section "AllGather KV" (a query slice attends over the
 * full sequence), section "Ring Attention" (key/value chunks arrive one at a
 * time and an online softmax folds each into the output, so the full K and V
 * are never materialised), and section "DeepSpeed Ulysses" (full-sequence
 * attention on a subset of heads).  Section "Context parallelism" fixes the
 * attention as bidirectional.
 *
 * For query row i of head (b, h) and the keys j of one chunk:
 *     s_ij = scale * <Q[b,h,i,:], K[b,h,j,:]>,  m_i = max_j s_ij,
 *     l_i  = sum_j exp(s_ij - m_i),
 *     O[b,h,i,:] = sum_j exp(s_ij - m_i) / l_i * V[b,h,j,:],
 *     LSE[b,h,i] = m_i + ln(l_i)               (natural log, scale included).
 * Two results over disjoint key sets merge exactly:
 *     LSE = ln(exp(LSE_1) + exp(LSE_2)),
 *     O   = exp(LSE_1 - LSE) * O_1 + exp(LSE_2 - LSE) * O_2.
 *
 * Conventions (shared by every entry point):
 *  - Tensors are [B, H, S, D] with the d index contiguous (stride 1); the b,
 *    h and s strides are given in ELEMENTS by attn_strides_t, so [B, S, H, D]
 *    views work too.  LSE tensors are [B, H, Sq] fp32, contiguous.
 *  - Every tensor pointer is a DEVICE pointer, 16-byte aligned; every stride
 *    times the element size must be a multiple of 16 bytes.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the legacy default stream).  Nothing is synchronised by the library.
 *  - The caller owns every buffer.  The library allocates no device memory
 *    (apart from the static scratch array of attn_shard_fwd_noalloc, part of
 *    the library's code object) and is re-entrant.  It keeps no state from
 *    one call to the next beyond what it sets up once per device, thread-
 *    safely: that a kernel's LDS size attribute is set, and the scratch
 *    array's device address.
 *  - Arguments are checked before anything is launched.  A non-OK status
 *    means nothing was enqueued and no output was touched, except
 *    ATTN_ERR_HIP, which reports a failed launch (a later kernel fault shows
 *    up, as in HIP, at the caller's next synchronisation).  No C++ exception
 *    crosses this interface.
 *  - Edge cases: Sq == 0 is a no-op returning ATTN_OK.  A chunk with no keys
 *    yields O = 0 and LSE = -inf.  Merging parts whose LSE are all -inf
 *    yields O = 0 and LSE = -inf (no NaN).  Non-finite inputs propagate.
 *  - Supported: D in {64, 128}; input dtype bf16 (MFMA path, fp32
 *    accumulation) or fp32 (fp32 throughout); output dtype bf16 or fp32 for
 *    bf16 inputs, fp32 for fp32 inputs.  For bf16 inputs one head's key and
 *    value rows must span less than 2 GiB: (Skv + 64) * s-stride * 2 bytes
 *    < 2^31 (ATTN_ERR_UNSUPPORTED otherwise).
 */
#ifndef LSDIT_ATTN_H
#define LSDIT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 1

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
    ATTN_ERR_SHAPE = 2,       /* negative size, chunk lengths not summing, order not a permutation */
    ATTN_ERR_DTYPE = 3,       /* unsupported dtype combination */
    ATTN_ERR_ALIGN = 4,       /* pointer or stride not 16-byte aligned, or d stride not 1 */
    ATTN_ERR_UNSUPPORTED = 5, /* head dimension other than 64 or 128, too many chunks */
    ATTN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than attn_shard_workspace_size() */
    ATTN_ERR_HIP = 7,         /* a kernel launch failed */
    ATTN_STATUS_MAX_ENUM = 0x7FFFFFFF /* not a status: makes any int32 a valid value of the type */
} attn_status_t;

typedef enum {
    ATTN_F32 = 0,
    ATTN_BF16 = 1,
    ATTN_DTYPE_MAX_ENUM = 0x7FFFFFFF /* not a dtype: any int32 is a valid value (and rejected) */
} attn_dtype_t;

/* Element strides of the b, h and s indices; the d stride is always 1. */
typedef struct {
    int64_t b, h, s;
} attn_strides_t;

/* An opaque hipStream_t. */
typedef void* attn_stream_t;

/* Most chunks attn_shard_fwd accepts, and most parts one attn_lse_merge call accepts. */
#define ATTN_MAX_CHUNKS 64

/* Merge modes of attn_shard_fwd (exactly one). */
#define ATTN_MERGE_NWAY 1u   /* every chunk writes an fp32 partial; one n-way merge at the end */
#define ATTN_MERGE_ONLINE 2u /* ring style: each chunk's kernel folds its result into a running fp32 result */
#define ATTN_MERGE_FUSED 4u  /* one kernel walks all chunks in order, the online-softmax state in registers */

/*
 * attn_chunk_fwd — attention of every query row against ONE chunk of keys.
 * (Blog sections "Ring Attention" and "AllGather KV": the per-rank, per-chunk
 * attention whose output the online softmax later folds together.)
 *
 *   q        [B, H, Sq, D] in_dt, strides qs
 *   k, v     [B, H, Skv, D] in_dt, strides ks, vs (the chunk's rows only)
 *   scale    softmax scale (1/sqrt(D) for standard attention), finite, > 0
 *   o        [B, H, Sq, D] o_dt, strides os: the chunk's output, normalised by
 *            the chunk's own row sum (an fp32 "partial" when o_dt = ATTN_F32)
 *   lse      [B, H, Sq] fp32 contiguous: the chunk's natural-log LSE
 * o and lse must not overlap q, k or v.
 */
attn_status_t attn_chunk_fwd(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks, const void* v,
                             attn_strides_t vs, attn_dtype_t in_dt, int32_t B, int32_t H, int32_t Sq, int32_t Skv,
                             int32_t D, float scale, void* o, attn_strides_t os, attn_dtype_t o_dt, float* lse,
                             attn_stream_t stream);

/*
 * attn_lse_merge — merge n results over disjoint key sets, row by row.
 * (Blog section "Ring Attention": each arriving key/value block updates the
 * attention output through the online softmax; this is that update, for any
 * number of blocks at once.)
 *
 *   o_parts, lse_parts   HOST arrays of n DEVICE pointers; part c is
 *                        [B, H, Sq, D] fp32 contiguous and [B, H, Sq] fp32.
 *   o_out                [B, H, Sq, D] o_dt, strides os (element strides,
 *                        so the merged output can go straight into a view
 *                        such as [B, S, H, D] storage)
 *   lse_out              [B, H, Sq] fp32 contiguous
 * 1 <= n <= ATTN_MAX_CHUNKS.  With o_dt = ATTN_F32 and contiguous strides,
 * o_out may alias o_parts[0] and lse_out may alias lse_parts[0] (the ring's
 * in-place online merge); no other overlap is allowed.  Parts with LSE -inf
 * carry no weight; a NaN LSE in any part makes the row's O and LSE NaN (as
 * attention over all the keys in one pass gives for a NaN query row).
 */
attn_status_t attn_lse_merge(int32_t n, const float* const* o_parts, const float* const* lse_parts, int32_t B,
                             int32_t H, int32_t Sq, int32_t D, void* o_out, attn_strides_t os, attn_dtype_t o_dt,
                             float* lse_out, attn_stream_t stream);

/*
 * attn_shard_workspace_size — bytes of device workspace attn_shard_fwd uses
 * for this shape, chunk count and merge mode: first the chunk slots, fp32
 * results [B,H,Sq,D] plus their LSE [B,H,Sq] (each part 256-byte aligned):
 * n of them for ATTN_MERGE_NWAY, one (the running result) for
 * ATTN_MERGE_ONLINE, none for ATTN_MERGE_FUSED or when n_chunks == 1.  Then,
 * for a shape of more than one round of query tiles (256 rows each) on the
 * current device's CUs, 4 KiB of work-queue counters (see attn_shard_fwd);
 * then, for a shape whose query tiles leave the last round part-full, room
 * for the balanced tail: (R * CUs + n_tail) slots of 256 * (D + 1) fp32
 * values, n_tail the query tiles of the last round, R = 4 when there is
 * more than one round, else 1 (nothing when the tiles fill whole rounds).
 * The slots are required; the room after them is optional (without it,
 * whole query tiles throughout, one workgroup each).
 * Returns 0 as well for invalid arguments; attn_shard_fwd reports those.
 */
size_t attn_shard_workspace_size(int32_t B, int32_t H, int32_t Sq, int32_t D, int32_t n_chunks, uint32_t flags);

/*
 * attn_shard_fwd — one GPU's share: its query rows against the whole key
 * sequence, processed chunk by chunk in the given order, the ring's chunk
 * loop run locally (blog sections "Ring Attention", "AllGather KV",
 * "DeepSpeed Ulysses").
 *
 *   q          [B, H, Sq, D] in_dt, strides qs
 *   k, v       [B, H, Skv, D] in_dt, strides ks, vs, Skv = sum of chunk_len
 *   chunk_len  HOST array of n_chunks lengths >= 0; chunk c covers key rows
 *              [off_c, off_c + chunk_len[c]) with off_c = sum_{c' < c} chunk_len[c']
 *   order      HOST permutation of 0..n_chunks-1 giving the processing order,
 *              or NULL for 0, 1, ..., n_chunks-1
 *   flags      one of ATTN_MERGE_NWAY, ATTN_MERGE_ONLINE, ATTN_MERGE_FUSED
 *              (ignored when n_chunks == 1).  FUSED is the ring's loop without
 *              partials: one kernel folds chunk after chunk into its running
 *              max, sum and output.  When its query tiles (bf16, 256 rows)
 *              leave the last round of CUs part-full and the keys are many,
 *              that round's work is spread evenly instead: each CU takes an
 *              equal run of (query tile, key tile) pairs, and a second kernel
 *              merges the runs' fp32 partials by their LSE (the balanced tail;
 *              only with the workspace: none given, whole tiles throughout).
 *              A bf16 launch of several rounds of query tiles and at least
 *              512 key tiles of work per CU runs persistent: one workgroup
 *              per CU takes whole query tiles, then the tail's runs (up to
 *              4 per CU, each at least 128 key tiles), from per-XCD work
 *              queues in the workspace, so that the XCDs end together
 *              whatever their clocks.  Which workgroup takes an item does
 *              not change the result.
 *              ONLINE and NWAY run one kernel per chunk
 *              (each with the balanced tail when it pays).  ONLINE is the
 *              ring's step: each chunk's kernel folds its result into the
 *              running fp32 result by the LSE rule in its epilogue (the last
 *              one into o and lse).  NWAY writes each chunk's fp32 partial and
 *              merges them all at the end with attn_lse_merge's kernel.
 *   workspace  DEVICE buffer, 16-byte aligned, of attn_shard_workspace_size()
 *              bytes; at least its chunk slots are required
 *              (ATTN_ERR_WORKSPACE otherwise), the tail's room after them is
 *              used when present (may be NULL when no slots are needed)
 *   o, lse     as in attn_chunk_fwd, for the whole key sequence
 * 1 <= n_chunks <= ATTN_MAX_CHUNKS.  The result equals attention over all
 * Skv keys up to rounding, whatever the chunking and order.
 */
attn_status_t attn_shard_fwd(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks, const void* v,
                             attn_strides_t vs, attn_dtype_t in_dt, int32_t B, int32_t H, int32_t Sq, int32_t D,
                             float scale, int32_t n_chunks, const int32_t* chunk_len, const int32_t* order,
                             uint32_t flags, void* workspace, size_t ws_bytes, void* o, attn_strides_t os,
                             attn_dtype_t o_dt, float* lse, attn_stream_t stream);

/*
 * attn_shard_fwd_noalloc — attn_shard_fwd with the ATTN_MERGE_FUSED schedule
 * and no workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc.  It calls no hipMalloc, hipFree or other allocating routine.
 *
 * The balanced tail's fp32 partials (see attn_shard_fwd) go to a scratch
 * array in the library's static device memory instead of a workspace:
 * ATTN_NOALLOC_SCRATCH_BYTES bytes (2 * 256 * 256 * (128 + 1) fp32 values,
 * 64.5 MiB) on each device the library runs on, held until the process ends.
 * The tail's plan spreads over at most 256 workgroups, so the need never
 * exceeds it for D <= 128; a shape that would need more is rejected with
 * ATTN_ERR_WORKSPACE before anything is launched.
 *
 * The first call on a device looks up that device's copy of the array (the
 * set-up; a caller that captures graphs makes one call before capturing).
 * Every call on a device shares its one array, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one
 * device (two streams, or two threads) race on it and must be serialised by
 * the caller.  Arguments, results and errors are those of attn_shard_fwd with
 * flags = ATTN_MERGE_FUSED.  It launches one workgroup per item with at most
 * one tail run per CU (never persistent), so on a device of at most 256 CUs
 * its result is bitwise that of attn_shard_fwd with a workspace of
 * attn_shard_workspace_size() bytes for the launches attn_shard_fwd does not
 * run persistent; for the others attn_shard_fwd may cut the tail into more
 * runs, and the two agree to fp32 rounding.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES 67633152u
attn_status_t attn_shard_fwd_noalloc(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks,
                                     const void* v, attn_strides_t vs, attn_dtype_t in_dt, int32_t B, int32_t H,
                                     int32_t Sq, int32_t D, float scale, int32_t n_chunks, const int32_t* chunk_len,
                                     const int32_t* order, void* o, attn_strides_t os, attn_dtype_t o_dt, float* lse,
                                     attn_stream_t stream);

/*
 * attn_ulysses_pack / attn_ulysses_unpack — the local halves of the all-to-all
 * around DeepSpeed-Ulysses attention (blog section "DeepSpeed Ulysses": each
 * rank trades its sequence slice of all heads for the whole sequence of a
 * subset of heads, and trades back after attention).
 *
 *   pack:   packed[j][s][b][h'][d] = x[b][j*Hg + h'][s][d]
 *   unpack: x[b][j*Hg + h'][s][d]  = packed[j][s][b][h'][d]
 *
 *   x       [B, H, S, D] in dt, strides xs (d stride 1): a rank's sequence
 *           slice, or on one GPU the whole sequence
 *   packed  [n][S][B][Hg][D] in dt, contiguous, Hg = H / n: part j is what
 *           goes to (pack) or came from (unpack) rank j
 *   dt      ATTN_BF16 or ATTN_F32; n >= 1 with H % n == 0
 * Because each part is in [S, B, Hg, D] order, the parts rank j receives from
 * ranks 0..n-1 (consecutive sequence slices) concatenate into head group j over
 * the whole sequence, which attn_chunk_fwd and attn_shard_fwd read as a strided
 * [B, Hg, S_total, D] view: b stride Hg*D, h stride D, s stride B*Hg*D.  On one
 * GPU, packing the whole sequence gives every head group's input directly.
 * x and packed must not overlap.  Same pointer/stride alignment rules and
 * error behaviour as the other entry points; S = 0 or B = 0 is a no-op.
 */
attn_status_t attn_ulysses_pack(const void* x, attn_strides_t xs, attn_dtype_t dt, int32_t B, int32_t H, int32_t S,
                                int32_t D, int32_t n, void* packed, attn_stream_t stream);
attn_status_t attn_ulysses_unpack(const void* packed, attn_dtype_t dt, int32_t B, int32_t H, int32_t S, int32_t D,
                                  int32_t n, void* x, attn_strides_t xs, attn_stream_t stream);

/*
 * attn_chunk_fwd_fp8 — the FP8 variant of attn_chunk_fwd: attention of every
 * query row against one chunk of keys, on OCP FP8 E4M3 inputs (8-bit floats,
 * which suit attention layers: page "TensorRT Multi-Device Inference:
 * Engineering Practices for Breaking Through Single-GPU Memory Bottlenecks",
 * section "Why a Single GPU Is No Longer Enough").
 *
 *   q, k, v  E4M3 codes, one byte per element, [B,H,Sq,D] / [B,H,Skv,D] with
 *            strides qs, ks, vs in elements (= bytes), d stride 1; the values
 *            are code * q_descale (k_descale, v_descale), descales finite > 0
 *   D        128 only (else ATTN_ERR_UNSUPPORTED)
 *   o, lse   as attn_chunk_fwd: O in o_dt (ATTN_BF16 or ATTN_F32), natural-log
 *            LSE fp32 [B,H,Sq] contiguous, scale included
 *   workspace  device scratch of at least attn_fp8_workspace_size(B,H,Sq,Skv,D)
 *            bytes, 16-byte aligned, owned by the caller; it receives V
 *            re-laid out as transposed 64-key tiles and, when the query tiles
 *            (256 rows) leave the last round of CUs part-full and the keys
 *            are many, the fp32 partials of the balanced tail (as in
 *            attn_shard_fwd); it may be reused once the call's work on
 *            `stream` has finished
 * The probabilities enter P.V as E4M3 (after scaling by 2^5), so the result
 * differs from exact attention of the decoded inputs by up to 2^-4 of the
 * probability-weighted mean of |V| per element (relative rounding of each
 * probability); the row sum adds the same rounded probabilities.
 * Pointers must be 16-byte aligned and b/h/s strides multiples of 16 bytes
 * (ATTN_ERR_ALIGN); one head's K rows must span under 2 GiB and Skv < 2^23
 * (ATTN_ERR_UNSUPPORTED); a short workspace gives ATTN_ERR_WORKSPACE.
 * Sq = 0, B = 0 or H = 0 is a no-op; Skv = 0 gives O = 0, LSE = -inf.
 */
size_t attn_fp8_workspace_size(int32_t B, int32_t H, int32_t Sq, int32_t Skv, int32_t D);
attn_status_t attn_chunk_fwd_fp8(const void* q, attn_strides_t qs, const void* k, attn_strides_t ks, const void* v,
                                 attn_strides_t vs, float q_descale, float k_descale, float v_descale, int32_t B,
                                 int32_t H, int32_t Sq, int32_t Skv, int32_t D, float scale, void* workspace,
                                 size_t ws_bytes, void* o, attn_strides_t os, attn_dtype_t o_dt, float* lse,
                                 attn_stream_t stream);

/* Static, human-readable name of a status code. */
const char* attn_status_str(attn_status_t s);

/* ATTN_ABI_VERSION of the built library. */
int32_t attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSDIT_ATTN_H */
