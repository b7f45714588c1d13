/*
 * gvattn -- segmented ("gapped") variable-length attention forward, LSE
 * merge and gradients for AMD Instinct MI355X (gfx950).  Plain C ABI:
 * pointers and sizes only, no C++ or framework types.
 *
 * The operation (the sources are the pages this library implements):
 *
 *   cosmos-framework PR #302 ("gapped replay on GPUs FlashAttention-4 has no
 *   kernels for"), section "What": Q, K and V are packed segment after
 *   segment.  Segment s owns query rows [cu_q[s], cu_q[s+1]) and key rows
 *   [cu_k[s], cu_k[s+1]) (its capacities) and uses only the prefixes of
 *   length seqused_q[s] and seqused_k[s].  The used query rows of a segment
 *   attend the used keys of the same segment only.  Rows past a segment's
 *   used length are left as they are, and a segment with no keys gets a zero
 *   output and a -inf log-sum-exp.
 *
 *   TensorRT-LLM issue #18687 ("Cosmos3 sequence-parallel path attends
 *   zero-padded text K/V"), sections "actual behavior" and "additional
 *   notes": keys past the used length are excluded by a key-padding mask,
 *   never merely zeroed, because a zero key would add exp(0) = 1 to the
 *   softmax denominator.
 *
 *   cosmos-framework PR #312 ("support SM120 replay with dense FA4
 *   batches"), section "Problem and behavior": GQA folding, FP32 LSE, and
 *   an FP32 LSE merge that combines the partial results of several
 *   visibility partitions.
 *
 * Conventions (readings of what the pages leave open):
 *   - query head h reads KV head h / (hq / hkv);
 *   - causal masks are aligned bottom-right inside each segment: query row i
 *     (0-based in the segment) sees key j iff j <= i + seqused_k - seqused_q;
 *   - any row with no visible key (an empty segment, or a causal row above
 *     the diagonal when seqused_k < seqused_q) gets O = +0 and LSE = -inf;
 *   - LSE is the natural logarithm of sum_j exp(softmax_scale * q.k_j);
 *   - layouts (row-major, innermost last):
 *       Q   [total_q, hq,  d]      K [total_k, hkv, d]     V [total_k, hkv, d_v]
 *       O   [total_q, hq,  d_v]    LSE float [hq, total_q]
 *     Q, K, V and O share one element type (gvattn_dtype); LSE is fp32.
 *
 * Ownership and streams: every buffer is caller-owned device memory.  The
 * library never allocates, frees, copies between host and device or
 * synchronises (except gvattn_read_device_error, which is a debugging aid).
 * All work is enqueued on `hip_stream` (a hipStream_t; NULL is the null
 * stream) in argument order.  Calls on one workspace must not overlap.
 *
 * Errors: every host-checkable problem returns a status code before any
 * work is enqueued.  Problems that depend on device data (a used length
 * beyond its capacity, offsets out of range or decreasing, a segment that
 * spans 2 GiB or more) cannot be seen without a synchronisation: the plan
 * kernel skips such a segment (its rows are left untouched) and sets a bit
 * in the workspace's device error word, which gvattn_read_device_error
 * returns.
 */
#ifndef GVATTN_H
#define GVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gvattn_status {
  GVATTN_OK = 0,
  GVATTN_ERR_INVALID_ARG = 1,  /* null pointer, negative size, hq % hkv != 0, bad scale ... */
  GVATTN_ERR_UNSUPPORTED = 2,  /* head dim, dtype or partition count not built */
  GVATTN_ERR_WORKSPACE = 3,    /* workspace missing, misaligned or too small */
  GVATTN_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} gvattn_status;

typedef enum gvattn_dtype {
  GVATTN_FP32 = 0,
  GVATTN_BF16 = 1,
  GVATTN_FP16 = 2
} gvattn_dtype;

/* Device error word bits (see gvattn_read_device_error). */
#define GVATTN_DEVERR_USED_Q 1   /* seqused_q[s] < 0 or > cu_q[s+1]-cu_q[s]  */
#define GVATTN_DEVERR_USED_K 2   /* seqused_k[s] < 0 or > cu_k[s+1]-cu_k[s]  */
#define GVATTN_DEVERR_OFFSETS 4  /* cu_* decreasing, negative or past total_* */
#define GVATTN_DEVERR_RANGE 8    /* a segment's rows span 2 GiB or more      */
#define GVATTN_DEVERR_PLAN 16    /* gvattn_fwd_run found no matching plan   */
#define GVATTN_DEVERR_KRANGES 32 /* key ranges: kr_off out of order or past
                                    nranges, a range outside [0, total_k),
                                    a negative length, 2^31 keys or more  */

/* Largest partition count gvattn_lse_merge accepts. */
#define GVATTN_MAX_PARTS 8

/* Alignment the workspace pointer must have, in bytes. */
#define GVATTN_WORKSPACE_ALIGN 256

/*
 * Bytes of device workspace gvattn_fwd needs for this geometry: a plan
 * header, the work list and per-segment offsets, and, for launches with few
 * query tiles (fewer than 512 tiles x head groups, 16-bit types), room for
 * FP32 split-K partials: up to 16 chunks of [total_q, hq, d_v] plus their
 * LSE, 64 MiB at most.  It depends only on the host-known sizes, never on
 * device data.
 * Returns 0 for invalid arguments.
 */
size_t gvattn_fwd_workspace_size(int32_t nseg, int32_t total_q, int32_t hq,
                                 int32_t hkv, int32_t d, int32_t d_v, int32_t dtype);

/*
 * Segmented varlen attention forward: plan + run (PR #302, "What").
 *
 *   dtype            GVATTN_BF16 or GVATTN_FP16 (matrix-core path, fp32
 *                    accumulation, P and O rounded to nearest even) or
 *                    GVATTN_FP32 (vector path).
 *   q, k, v          device, layouts above; may hold anything (NaN
 *                    included) in gap rows, which are never read into a
 *                    result.
 *   cu_seqlens_q/k   device int32 [nseg + 1], segment start offsets; the
 *                    last entry bounds the last segment's capacity.
 *                    Segments may leave rows between them.
 *   seqused_q/k      device int32 [nseg], used prefix of each segment.
 *   nseg             >= 0 (0 is a no-op).
 *   total_q/total_k  rows of the Q/O and K/V buffers.
 *   hq, hkv          heads, hq % hkv == 0.
 *   d                head dim of Q and K: 64, 128 or 256.
 *   d_v              head dim of V and O: 64, 128 or 256 (may differ from d;
 *                    the pages' FA2 path requires equal dims and sends the
 *                    rest to an FP32 fallback, PR #302 review).
 *   softmax_scale    finite and > 0 (typically 1/sqrt(d)).
 *   causal           0 or 1 (bottom-right within each segment).
 *   out, lse         device, written for used rows only; every other row is
 *                    left bit-for-bit as it was.  Must not overlap q/k/v.
 *   workspace        device, GVATTN_WORKSPACE_ALIGN-aligned, at least
 *                    gvattn_fwd_workspace_size(...) bytes.
 *   hip_stream       hipStream_t to enqueue on.
 */
int gvattn_fwd(int32_t dtype, const void* q, const void* k, const void* v,
               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
               const int32_t* seqused_q, const int32_t* seqused_k,
               int32_t nseg, int32_t total_q, int32_t total_k,
               int32_t hq, int32_t hkv, int32_t d, int32_t d_v,
               float softmax_scale, int32_t causal,
               void* out, float* lse,
               void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * The two halves of gvattn_fwd, for callers that replay one geometry many
 * times: the segment lengths are then read once, by the plan, instead of at
 * every launch (the PR #302 review asks for segment geometry that is not
 * read back to the host on every call).
 *
 * gvattn_fwd_plan reads only the geometry arrays and writes the sorted tile
 * work list into the workspace.  gvattn_fwd_run takes the same arguments as
 * gvattn_fwd and runs the attention on the plan found in the workspace; the
 * geometry arrays must hold the values the plan was built from.  A plan
 * built for any other host-side geometry (element type's tile shape, hq,
 * hkv, d, d_v, causal flag, segment count, total_q, total_k or workspace
 * layout) is detected on the device: the run writes nothing and sets
 * GVATTN_DEVERR_PLAN.
 */
int gvattn_fwd_plan(int32_t dtype,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    const int32_t* seqused_q, const int32_t* seqused_k,
                    int32_t nseg, int32_t total_q, int32_t total_k,
                    int32_t hq, int32_t hkv, int32_t d, int32_t d_v, int32_t causal,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

int gvattn_fwd_run(int32_t dtype, const void* q, const void* k, const void* v,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                   const int32_t* seqused_q, const int32_t* seqused_k,
                   int32_t nseg, int32_t total_q, int32_t total_k,
                   int32_t hq, int32_t hkv, int32_t d, int32_t d_v,
                   float softmax_scale, int32_t causal,
                   void* out, float* lse,
                   void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Forward over key ranges (TensorRT-LLM issue #18687, "additional notes",
 * first of the possible fixes: the Ulysses exchange leaves keys ordered by
 * rank, so a sample's valid keys are several runs of rows rather than one
 * prefix).  Plan + attention in one call, as gvattn_fwd.
 *
 * Segment s's keys are the concatenation, in list order, of the K/V row
 * ranges [kr_start[i], kr_start[i] + kr_len[i]) for i in [kr_off[s],
 * kr_off[s + 1]).  Everything else is gvattn_fwd with seqused_k[s] = the
 * total length of those ranges; the bottom-right causal alignment counts
 * keys in the concatenated order.  A range may repeat or overlap another
 * (each listed row is one key per listing).
 *
 *   kr_off         device int32 [nseg + 1], non-decreasing, within
 *                  [0, nranges].
 *   kr_start, kr_len  device int32 [nranges]; 0 <= kr_start, 0 <= kr_len,
 *                  kr_start + kr_len <= total_k.  May be NULL when
 *                  nranges == 0.
 *   workspace      gvattn_fwd_workspace_size(...) bytes, as for gvattn_fwd.
 *   other arguments as for gvattn_fwd (no cu_seqlens_k / seqused_k).
 * A segment whose ranges break these rules is skipped (its rows are left
 * untouched) and GVATTN_DEVERR_KRANGES is set in the workspace error word.
 */
int gvattn_fwd_ranges(int32_t dtype, const void* q, const void* k, const void* v,
                      const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                      const int32_t* kr_off, const int32_t* kr_start,
                      const int32_t* kr_len, int32_t nseg, int32_t nranges,
                      int32_t total_q, int32_t total_k,
                      int32_t hq, int32_t hkv, int32_t d, int32_t d_v,
                      float softmax_scale, int32_t causal,
                      void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * gvattn_fwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * gvattn_fwd, minus `workspace` / `workspace_bytes`.  The plan (and any
 * split-K partials) goes to a static device array of
 * GVATTN_NOALLOC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends; nothing is allocated or freed.  When the
 * ordinary split-K partials do not fit, fewer key chunks are used (same
 * results within the stated tolerances); a geometry whose plan alone does
 * not fit returns GVATTN_ERR_WORKSPACE before anything is enqueued.
 * All calls on one device share the array: calls that may overlap on one
 * device (different streams, or threads without ordering) race and must
 * be serialised by the caller.  The array needs no clearing: every call
 * writes the plan it reads.
 */
#define GVATTN_NOALLOC_SCRATCH_BYTES 33554432 /* 32 MiB */

int gvattn_fwd_noalloc(int32_t dtype, const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       const int32_t* seqused_q, const int32_t* seqused_k,
                       int32_t nseg, int32_t total_q, int32_t total_k,
                       int32_t hq, int32_t hkv, int32_t d, int32_t d_v,
                       float softmax_scale, int32_t causal,
                       void* out, float* lse, void* hip_stream);

/*
 * FP32 LSE merge of nparts partial results over key partitions (PR #312,
 * "Problem and behavior").  For every used row (rows [cu_seqlens_q[s],
 * cu_seqlens_q[s] + seqused_q[s])) and head, in FP32:
 *   m = max_p LSE_p;  m = -inf  ->  O = 0, LSE = -inf;
 *   otherwise w_p = exp(LSE_p - m), W = sum_p w_p,
 *             LSE = m + ln W,  O = sum_p (w_p / W) O_p.
 * A NaN in any LSE_p makes that row's O and LSE NaN.  Gap rows are left
 * untouched.
 *
 *   nparts         1 .. GVATTN_MAX_PARTS.
 *   part_out       HOST array of nparts device pointers, each
 *                  [total_q, hq, d] of part_dtype.
 *   part_lse       HOST array of nparts device pointers, each fp32
 *                  [hq, total_q].
 *   part_dtype     element type of the partial outputs (any gvattn_dtype).
 *   out_dtype      element type of `out` (any gvattn_dtype).
 *   cu_seqlens_q   device int32 [nseg + 1]; seqused_q device int32 [nseg].
 *   out, lse       device; `out` may be part_out[0] when out_dtype equals
 *                  part_dtype, and `lse` may be part_lse[0] (each row and
 *                  head is read completely before it is written); no other
 *                  overlap.  out == part_out[0] with differing element
 *                  types is GVATTN_ERR_INVALID_ARG.
 *   device_error   optional device int32; invalid segments are skipped and
 *                  GVATTN_DEVERR_* bits are OR-ed into it.  May be NULL.
 */
int gvattn_lse_merge(int32_t nparts, const void* const* part_out,
                     const float* const* part_lse, int32_t part_dtype,
                     int32_t out_dtype,
                     const int32_t* cu_seqlens_q, const int32_t* seqused_q,
                     int32_t nseg, int32_t total_q, int32_t hq, int32_t d,
                     void* out, float* lse, int32_t* device_error,
                     void* hip_stream);

/* Static text for a gvattn_status value. */
const char* gvattn_status_string(int status);

/*
 * Bytes of device workspace gvattn_bwd needs: two plans (query tiles for
 * dQ, 64-key tiles for dK / dV), 8 bytes of per-row statistics per (query
 * head, query row) and FP32 partials for launches with few key tiles (at
 * most 1024 x 64 x (d + d_v) x 4 bytes).  Depends only on host-known sizes.
 * Returns 0 for invalid or unsupported arguments.
 */
size_t gvattn_bwd_workspace_size(int32_t nseg, int32_t total_q, int32_t total_k,
                                 int32_t hq, int32_t hkv, int32_t d, int32_t d_v,
                                 int32_t dtype);

/*
 * Gradients of gvattn_fwd with respect to Q, K and V.  The pages' path is
 * forward-only (PR #302, review: its backward raises); this is the plain
 * calculus of the forward they define (PR #302, "What"; PR #312, "Problem
 * and behavior").  Per segment and query head h (KV head g = h / (hq/hkv)),
 * with P = exp(softmax_scale * Q K^T - LSE) over the used rows and the keys
 * each row sees, and D = rowsum(dO * O):
 *   dV_g = sum_h P^T dO,   dS = P * (dO V^T - D),
 *   dQ   = softmax_scale * dS K,   dK_g = softmax_scale * sum_h dS^T Q.
 *
 *   dtype            GVATTN_BF16 or GVATTN_FP16 (fp32 accumulation; P and
 *                    dS rounded to nearest even for the matrix cores).
 *                    GVATTN_FP32 returns GVATTN_ERR_UNSUPPORTED.
 *   q, k, v          the forward's inputs (layouts above).
 *   out, lse         the forward's outputs for the same inputs: O
 *                    [total_q, hq, d_v], LSE fp32 [hq, total_q].  Only
 *                    used rows are read.
 *   dout             dL/dO, [total_q, hq, d_v], dtype.  Only used rows are
 *                    read.
 *   cu_seqlens_*, seqused_*, nseg, total_*, hq, hkv, softmax_scale, causal
 *                    as in gvattn_fwd (the key-prefix form).
 *   d, d_v           64 or 128 each (others: GVATTN_ERR_UNSUPPORTED).
 *   dq               [total_q, hq, d]: written for used rows (0 for a row
 *                    that sees no key); other rows are left untouched.
 *   dk, dv           [total_k, hkv, d] and [total_k, hkv, d_v]: written for
 *                    the used keys of every segment (0 for a key no row
 *                    sees); other rows are left untouched.
 *                    dq, dk and dv must not overlap each other or any input.
 *   workspace        device, GVATTN_WORKSPACE_ALIGN-aligned, at least
 *                    gvattn_bwd_workspace_size(...) bytes.
 * Device-data errors are reported as for gvattn_fwd (the affected segment
 * is skipped; gvattn_read_device_error on this workspace).
 */
int gvattn_bwd(int32_t dtype, const void* q, const void* k, const void* v,
               const void* out, const void* dout, const float* lse,
               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
               const int32_t* seqused_q, const int32_t* seqused_k,
               int32_t nseg, int32_t total_q, int32_t total_k,
               int32_t hq, int32_t hkv, int32_t d, int32_t d_v,
               float softmax_scale, int32_t causal,
               void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Debugging aid: waits for `hip_stream`, then copies the device error word
 * of `workspace` (GVATTN_DEVERR_* bits of the last plan and the runs on it)
 * into *err_out.  Synchronises; not for the hot path.
 */
int gvattn_read_device_error(const void* workspace, void* hip_stream,
                             int32_t* err_out);

/* Library ABI version (major * 100 + minor). */
int gvattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GVATTN_H */
