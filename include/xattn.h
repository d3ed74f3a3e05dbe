/*
 * xattn.h -- C ABI of libxattn.so: fused causal scaled-dot-product attention,
 * forward and backward, for AMD Instinct MI355X (gfx950).
 *
 * The operation (after the fused attention kernel of the "xtrain evolution
 * overview" page, section 一 infra-phase table, row T14, and the batched
 * attention of the KI-1 fix on "xtrain -- Known Issues & Perf Backlog"):
 *
 *   For batch b, query head h, kv head g = h / (H / Hkv) (grouped-query
 *   attention as in row T15 of the same table: query head h reads kv head
 *   floor(h / group), no copy of K/V is made), and rows i, j < S:
 *
 *     s_ij  = scale * q_i . k_j                      (key j visible iff j <= i)
 *     P_ij  = exp(s_ij - LSE_i),  LSE_i = ln sum_{j<=i} exp(s_ij)
 *     o_i   = sum_{j<=i} P_ij v_j
 *
 *   and, for an upstream gradient dO, with D_i = sum_d dO_id o_id
 *   (the row-T14 simplification of the softmax Jacobian):
 *
 *     dS_ij = P_ij (dO_i . v_j - D_i)
 *     dq_i  = scale * sum_{j<=i} dS_ij k_j
 *     dk_j  = scale * sum_{h in group(g)} sum_{i>=j} dS_ij q_i
 *     dv_j  =         sum_{h in group(g)} sum_{i>=j} P_ij dO_i
 *
 *   The causal mask is top-left aligned (Sq == Sk == S).  No S x S buffer is
 *   ever allocated.
 *
 * Layout: every tensor is contiguous, head-major ("BHSD"):
 *   q, o, dO, dq : [B][H][S][hd]        k, v, dk, dv : [B][Hkv][S][hd]
 *   lse          : [B][H][S]            workspace    : see xattn_bwd_workspace_bytes
 *
 * Types: q, k, v, o, dO are XATTN_F32 (float) or XATTN_BF16 (bfloat16 bit
 *   patterns, 2 bytes).  lse, dq, dk, dv and the workspace are always float.
 *   In bf16 mode products are accumulated in fp32; softmax is fp32; the
 *   probabilities and dS are rounded to bf16 (nearest-even) before they enter
 *   a matrix product; o is rounded to bf16 (nearest-even).
 *
 * Ownership and execution: all pointers are DEVICE pointers owned by the
 *   caller.  The library never allocates, frees or synchronises, keeps no
 *   global state, and only enqueues kernels on `stream` (a hipStream_t; NULL
 *   means the legacy default stream) before returning.  Outputs are fully
 *   overwritten, never accumulated.  Inputs are never modified.  Outputs must
 *   not alias inputs or each other.  Device faults surface at the caller's next
 *   synchronisation, as with any asynchronous HIP call.
 *
 * Errors: every argument is validated on the host before any HIP call; an
 *   invalid call returns its status code and enqueues nothing.  A failed
 *   kernel launch returns XATTN_ERR_HIP.
 *
 * Supported: hd in {16, 32, 64}; any S >= 1; H a multiple of Hkv; scale a
 *   positive finite number; every data pointer 16-byte aligned; every tensor
 *   below 2^31 elements per (batch, head) plane; and every kernel launch a
 *   call makes within HIP's limit of 2^32 - 1 work-items, i.e. at most
 *   16777215 workgroups of 256 threads (the forward launches B*H*ceil(S/128)
 *   of them, the fp32 dq kernel B*H*ceil(S/64); larger shapes return
 *   XATTN_ERR_SHAPE before anything is enqueued).
 */
#ifndef XATTN_H
#define XATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  XATTN_F32 = 0,
  XATTN_BF16 = 1
} xattn_dtype;

typedef enum {
  XATTN_OK = 0,
  XATTN_ERR_NULL = 1,       /* a required pointer is NULL */
  XATTN_ERR_SHAPE = 2,      /* B, S, H, Hkv or hd <= 0, or a size limit exceeded */
  XATTN_ERR_GQA = 3,        /* H is not a multiple of Hkv */
  XATTN_ERR_HEAD_DIM = 4,   /* hd not in {16, 32, 64} */
  XATTN_ERR_DTYPE = 5,      /* dtype is not an xattn_dtype */
  XATTN_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than required */
  XATTN_ERR_SCALE = 7,      /* scale not positive and finite */
  XATTN_ERR_HIP = 8,        /* the HIP runtime rejected a kernel launch */
  XATTN_ERR_ALIGN = 9,      /* a data pointer is not 16-byte aligned */
  XATTN_ERR_PARAM = 10,     /* eps or rope base out of range (QK-norm + RoPE) */
  XATTN_ERR_SCRATCH = 11    /* too large for xattn_bwd_noalloc's fixed scratch */
} xattn_status;

/*
 * Forward (row T14 of the infra table: online softmax tiled over KV, the
 * per-row logsumexp kept for the backward).
 *   q [B][H][S][hd], k and v [B][Hkv][S][hd] in `dtype`  (inputs)
 *   o [B][H][S][hd] in `dtype`, lse [B][H][S] float      (outputs)
 *   lse is the natural-log logsumexp of the scaled, masked scores.
 * Returns an xattn_status.
 */
int xattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int S, int H, int Hkv, int hd, float scale, int dtype,
              void* stream);

/*
 * Bytes of device workspace xattn_bwd needs: 8*B*H*S (two floats per query
 * row: -D = -rowsum(dO * o) and LSE * log2(e)), O(B*H*S), never S x S.  For
 * grouped-query shapes with few kv tiles (B * Hkv * ceil(S/128) < 512) the
 * dk/dv kernel splits the query heads of each group into R slices (R the
 * least divisor of H/Hkv with R * B * Hkv * ceil(S/128) >= 1024 for fp32,
 * >= 512 for bf16, else H/Hkv), one workgroup each, and keeps their partial
 * dk, dv here too: the first part rounded up to a multiple of 16 bytes, plus
 * 8 * R * B * Hkv * S * hd bytes.
 * Returns 0 for invalid shapes.
 */
size_t xattn_bwd_workspace_bytes(int B, int S, int H, int Hkv, int hd, int dtype);

/*
 * Backward (row T14: scores recomputed from q, k and lse; D = rowsum(dO * o);
 * row T15: dk/dv summed over the query heads of each kv group in a fixed
 * order, no atomics, so results are bitwise reproducible run to run).
 *   q, o, dO [B][H][S][hd] and k, v [B][Hkv][S][hd] in `dtype`, lse [B][H][S]
 *   float (inputs; o and lse may come from any source, e.g. xattn_fwd)
 *   dq [B][H][S][hd], dk and dv [B][Hkv][S][hd] float (outputs)
 *   workspace: device scratch of at least xattn_bwd_workspace_bytes(...) bytes,
 *   16-byte aligned; its contents on entry do not matter.
 * Enqueues xattn_bwd_kernel_count(...) kernels in order on `stream`: for short
 * bf16 sequences one kernel computes dq, dk and dv and leaves the workspace
 * untouched; otherwise the dq kernel and the dk/dv kernel (plus a group-sum
 * kernel for split GQA groups).
 * Returns an xattn_status.
 */
int xattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, float* dq, float* dk, float* dv,
              int B, int S, int H, int Hkv, int hd, float scale, int dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of xattn_bwd, for callers that schedule them separately
 * (e.g. to overlap the query-side half with other work, or to time each).
 * xattn_bwd(...) gives bit for bit the results of xattn_bwd_dq(...) followed
 * on the same stream by xattn_bwd_dkdv(...) with the same arguments and
 * workspace; where xattn_bwd_kernel_count(...) is 2 or 3 it is exactly that
 * pair of calls, where it is 1 the same arithmetic runs in one kernel.
 *
 * xattn_bwd_dq: writes dq [B][H][S][hd] float and stores, per query row,
 *   -D = -rowsum(dO * o) and LSE * log2(e) in the workspace ([2][B][H][S] float).
 * xattn_bwd_dkdv: writes dk, dv [B][Hkv][S][hd] float; reads both per-row
 *   values from the workspace (not lse), so it must be ordered after an
 *   xattn_bwd_dq call with the same q, o, dO, lse, shapes and workspace; on
 *   grouped-query shapes it also writes partial sums past them (see
 *   xattn_bwd_workspace_bytes).
 * Argument meaning, layout, validation and status codes are those of xattn_bwd.
 */
/*
 * Number of kernels xattn_bwd enqueues for a shape (and xattn_bwd_ragged with
 * the same shape), 0 for an invalid one:
 *   1  dtype bf16, hd <= 32, S <= 256 and H == Hkv: one workgroup per
 *      (batch, head) holds the head's q, k, v and dO in LDS and computes D,
 *      dk, dv and then dq with the dq and dk/dv kernels' arithmetic (q, k, v,
 *      dO and o read from HBM once, one launch instead of two);
 *   2  xattn_bwd_dq, then xattn_bwd_dkdv;
 *   3  the same, with the dk/dv half's group sum (GQA groups split over
 *      workgroups, see xattn_bwd_workspace_bytes).
 * xattn_bwd_noalloc takes the same single kernel where this is 1, and the
 * pair of kernels otherwise (it never splits groups).  Host-only; touches no
 * device.
 */
int xattn_bwd_kernel_count(int B, int S, int H, int Hkv, int hd, int dtype);

int xattn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dO, float* dq, int B, int S, int H, int Hkv, int hd, float scale,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream);

int xattn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                   const void* dO, float* dk, float* dv, int B, int S, int H, int Hkv, int hd,
                   float scale, int dtype, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * xattn_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It allocates nothing (no hipMalloc, no allocating
 * library call): the per-row scratch (-D and LSE * log2(e), 8*B*H*S bytes)
 * lives in a fixed 16 MiB device array inside the library, one per GPU,
 * held from the first call on that GPU until the process ends.
 *   Arguments, layout, dtypes and the result are those of xattn_bwd, except
 *   that the query heads of a GQA group are never split over workgroups (the
 *   dk, dv group sum runs in one workgroup per key tile, in the same fixed
 *   order), so it needs no room for partial sums.
 *   Limit: 8*B*H*S <= 16777216 (B*H*S <= 2097152 query rows); larger shapes
 *   return XATTN_ERR_SCRATCH before anything is enqueued.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (e.g. on two streams without ordering between them) race and give
 *   wrong results.  Nothing in the array needs to start at zero (the first
 *   kernel writes every value the second reads).
 *   The first call on each GPU looks up the array's device address (no
 *   allocation, no synchronisation); make it outside a graph capture.
 * Returns an xattn_status.
 */
int xattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dO, float* dq, float* dk, float* dv,
                      int B, int S, int H, int Hkv, int hd, float scale, int dtype,
                      void* stream);

/*
 * Per-head RMS QK-norm + rotary position embedding: the step that turns a q (or
 * k) projection output into the attention input (the per-head QK-norm of the
 * "xtrain evolution overview", section 一, row T9; RoPE with the position
 * restarting per sequence, rows T5 and T10 and the KI-1 fix of "xtrain --
 * Known Issues & Perf Backlog"; the head-major transpose of that fix folded
 * into the store).  For token (b, s) and head h, x = X[b,s,h,:]:
 *   r = sqrt(mean_d x_d^2 + eps),  y = w * x / r,
 *   out[b,h,s,i]        = y_i cos t_i - y_{i+hd/2} sin t_i
 *   out[b,h,s,i+hd/2]   = y_{i+hd/2} cos t_i + y_i sin t_i,
 *   t_i = s * rope_base^(-2i/hd),  i < hd/2.
 *   x   [B][S][H][hd] in `dtype` (token-major, as the projection writes it)
 *   w   [hd] float (one weight per head dimension, shared by all heads)
 *   out [B][H][S][hd] in `dtype` (head-major: ready for xattn_fwd)
 * Norm arithmetic is fp32; bf16 outputs are rounded to nearest-even.
 * Supported: hd in {16, 32, 64}; B*S*H*hd < 2^31; eps finite >= 0; rope_base
 * finite > 1; 16-byte aligned pointers.  Same ownership, stream and error
 * rules as xattn_fwd.  Returns an xattn_status.
 */
int xattn_qknorm_rope_fwd(const void* x, const float* w, void* out, int B, int S, int H, int hd,
                          float eps, float rope_base, int dtype, void* stream);

/*
 * Bytes of device workspace xattn_qknorm_rope_bwd needs: hd floats per
 * workgroup of its fixed grid (at most 1024 workgroups, so at most 256 KB).
 * Returns 0 for invalid shapes.
 */
size_t xattn_qknorm_rope_bwd_workspace_bytes(int B, int S, int H, int hd);

/*
 * Backward of xattn_qknorm_rope_fwd for an upstream gradient dout:
 *   g = R(t)^T dout (the rotation transposed),  xh = x / r,  gxh = w * g,
 *   dx = (gxh - xh * mean_d(xh * gxh)) / r,   dw = sum over all (b, s, h) of xh * g.
 *   x    [B][S][H][hd] in `dtype`, w [hd] float          (inputs, as in the forward)
 *   dout [B][H][S][hd] float (e.g. xattn_bwd's dq or dk)  (input)
 *   dx   [B][S][H][hd] float, dw [hd] float               (outputs, overwritten)
 *   workspace: device scratch of at least xattn_qknorm_rope_bwd_workspace_bytes
 *   bytes, 16-byte aligned; its contents on entry do not matter.
 * dw is summed in a fixed order (no atomics): bitwise reproducible.  Two
 * kernels are enqueued in order on `stream`.  Returns an xattn_status.
 */
int xattn_qknorm_rope_bwd(const void* x, const float* w, const float* dout, float* dx, float* dw,
                          int B, int S, int H, int hd, float eps, float rope_base, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Right-padded batches with per-sequence lengths (the pad-and-mask batching of
 * the "xtrain evolution overview" page, post-training stage, milestone M2d:
 * sequences of different lengths are right-padded to one length S; under the
 * causal mask a real row never sees a later padding position, so its output
 * equals the unpadded sequence's).  Same operation, layout and rules as
 * xattn_fwd / xattn_bwd, plus
 *   lens  [B] int32 device array: sequence b holds rows 0 .. lens[b]-1 of its
 *         S-row planes (values clamped to [0, S] on the device).
 * For each sequence the result on its rows equals xattn_fwd / xattn_bwd of
 * that sequence alone (S = lens[b]); padding rows and keys are never read (they
 * may hold anything, NaN included) and are written as o = 0, lse = -inf,
 * dq = dk = dv = 0.  Work on tiles that hold only padding is skipped.
 * lens must be 4-byte aligned; it is required (NULL -> XATTN_ERR_NULL).
 * The workspace is the one xattn_bwd_workspace_bytes sizes.
 */
int xattn_fwd_ragged(const void* q, const void* k, const void* v, const int* lens, void* o,
                     float* lse, int B, int S, int H, int Hkv, int hd, float scale, int dtype,
                     void* stream);

int xattn_bwd_ragged(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, const int* lens, float* dq, float* dk, float* dv, int B,
                     int S, int H, int Hkv, int hd, float scale, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * The composed path: the same operation as xattn_fwd / xattn_bwd computed the
 * way the batched path of the KI-1 fix on "xtrain -- Known Issues & Perf
 * Backlog" does it (a batched Q.K^T, a causal softmax, then P.V, through an
 * S x S buffer per (batch, head); the fused kernel of row T14 of the "xtrain
 * evolution overview" infra table replaces it).  For comparing the two paths.
 *
 *   p   [B][H][S][S] float: forward output, backward input -- the causal
 *       probabilities P_ij (j <= i) in its lower triangle; entries past the
 *       diagonal up to the end of the row's 128-column tile are 0, the rest
 *       unspecified.  This buffer is the path's memory cost.
 *   ds  [B][H][S][S] float: backward scratch (dP, then dS), contents on entry
 *       irrelevant.
 * Both must hold at least xattn_composed_buffer_bytes(B, S, H) bytes (the
 * sizes are passed), 16-byte aligned.  Other arguments, layouts, dtypes and
 * rounding points as xattn_fwd / xattn_bwd.  Returns an xattn_status.
 */
size_t xattn_composed_buffer_bytes(int B, int S, int H);

int xattn_composed_fwd(const void* q, const void* k, const void* v, void* o, float* lse, float* p,
                       size_t p_bytes, int B, int S, int H, int Hkv, int hd, float scale,
                       int dtype, void* stream);

int xattn_composed_bwd(const void* q, const void* k, const void* v, const float* p,
                       size_t p_bytes, const void* dO, float* dq, float* dk, float* dv, float* ds,
                       size_t ds_bytes, int B, int S, int H, int Hkv, int hd, float scale,
                       int dtype, void* stream);

/*
 * Decode attention: the new query of each sequence against that sequence's
 * key/value cache (the decode-attention primitive of the "xtrain evolution
 * overview" page, post-training stage: milestone M2a -- one query against the
 * cached K/V, equal to the last row of full causal attention; M2b -- several
 * sequences decoded together, each with its own cache, GQA broadcasting each kv
 * head to its group; M2c -- the cache kept on the device, one [T, hd] plane per
 * (sequence, kv head)).  For sequence b holding n = lens[b] positions, query
 * head h, kv head g = h / (H / Hkv):
 *
 *   s_j = scale * q[b,h] . k[b,g,j]   (j < n),   lse[b,h] = ln sum_{j<n} exp(s_j),
 *   o[b,h] = sum_{j<n} exp(s_j - lse[b,h]) v[b,g,j]
 *
 * and for n = 0: o[b,h] = 0, lse[b,h] = -inf.  Positions j >= n are never read.
 *
 *   q, o    [B][H][hd]        in `dtype` (o overwritten; rounded to nearest-even in bf16)
 *   k, v    [B][Hkv][T][hd]   in `dtype`, T = cache capacity, at most 4194304 (inputs)
 *   lens    [B] int32 device array, or NULL (every sequence holds T positions).
 *           Values are clamped to [0, T] on the device (they cannot be checked on
 *           the host without a synchronisation).
 *   lse     [B][H] float, natural log, scale included (output)
 *   workspace: device scratch of at least xattn_decode_workspace_bytes bytes,
 *           16-byte aligned, contents on entry irrelevant; may be NULL when that
 *           size is 0.
 * Arithmetic is fp32 (bf16 inputs are widened exactly).  Long caches are split
 * into chunks handled by separate workgroups, merged by a second kernel in a
 * fixed order: bitwise reproducible run to run.  Same pointer, stream and error
 * rules as xattn_fwd (data pointers 16-byte aligned; lens 4-byte aligned).
 * Returns an xattn_status.
 */
size_t xattn_decode_workspace_bytes(int B, int T, int H, int Hkv, int hd);

int xattn_decode(const void* q, const void* k, const void* v, const int* lens, void* o,
                 float* lse, int B, int T, int H, int Hkv, int hd, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* xattn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H */
