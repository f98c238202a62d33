/*
 * attn_jvp.h -- fused softmax-attention forward pass and its Jacobian-vector
 * product (JVP) on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation.  The rCM record in the Anthology of the SOTA (LIT-783, "Key
 * takeaways", bullet "JVP at production scale", paper §3.2 and App. C)
 * credits a kernel that fuses the FlashAttention-2 forward with its
 * directional derivative in a single sweep over key tiles, whether the keys
 * come from the queries' own sequence or from another one, and with the
 * tangents of Q, K and V laid out like Q, K and V.  Per (batch b, head h), for
 * queries i < Nq, keys j < Nk, head dim d and the scalar `scale` s:
 *
 *   S   = s Q K^T,  P = row-softmax(S),  O = P V,
 *   lse = ln sum_j exp(S_ij)                                (natural log)
 *   dS  = s (dQ K^T + Q dK^T),  mu_i = sum_j P_ij dS_ij,
 *   dO  = (P * (dS - mu)) V + P dV                          (the tangent of O)
 *
 * `scale` is a constant: it has no tangent.  There is no mask, no causal
 * mode, no dropout and no grouped heads (K and V have H heads, like Q).
 *
 * Layout.  Every tensor is dense, row-major and contiguous:
 *   q, tq, o, to : [B, H, Nq, d]      k, v, tk, tv : [B, H, Nk, d]
 *   lse          : [B, H, Nq]
 * A tangent has exactly its primal's shape, dtype and layout.  The kernels
 * address every tensor through buffer descriptors that span exactly that
 * tensor, so an access outside it reads zero or is dropped.
 *
 * Sizes.  A descriptor takes 32-bit byte offsets, so one kernel launch covers
 * at most 2^31 bytes of each tensor.  Whole tensors may be larger: a call
 * whose tensors pass that runs as consecutive launches on `stream` over
 * groups of whole (b, h) slices, each group's tensors under 2^31 bytes (every
 * slice is independent and [B, H, N, d] keeps a group contiguous).  What stays
 * bounded is one slice of each tensor (see ATTN_JVP_EUNSUPPORTED).
 *
 * Precision.  attn_jvp_fwd takes bf16 inputs (uint16 storage holding IEEE
 * bfloat16 bit patterns); all products are formed on bf16/fp16 matrix cores
 * with fp32 accumulation, and O, dO and lse are written in fp32.  The second
 * contraction (P and s P dS against V and dV) runs on fp16 operands, kept
 * inside fp16's range by powers of two that are undone exactly in fp32: V and
 * dV are multiplied by 2^e per (b, h) slice, e chosen from the slice's largest
 * finite |V| (|dV|), so the conversion is exact apart from magnitudes below
 * 2^-29 of that largest one; s P dS is multiplied by 2^t per group of 32 query
 * rows, t chosen from an upper bound of |s dS| (Cauchy-Schwarz on the norms of
 * the rows of Q, dQ and the keys of K, dK), then rounded to nearest like P.
 * So every finite bf16 input is in range; what bounds the domain is fp32
 * itself: the logits s q.k, s dS and the results must be finite in fp32.
 * Scaling (V, dV) by a power of two scales O and dO by it exactly, and so does
 * scaling every tangent for dO and the tangent of lse.  attn_jvp_fwd_f32 takes
 * fp32 inputs and computes in fp32 throughout.  NaN and Inf inputs propagate:
 * an output is NaN or Inf where the exact result is (e.g. a NaN in row i of Q
 * or dQ reaches row i of the outputs only, a NaN in column c of V or dV column
 * c of O and dO).
 *
 * Ownership and streams.  All tensor pointers are DEVICE pointers owned by the
 * caller, on the current HIP device.  Outputs must not alias inputs or each
 * other.  Every call is asynchronous on `stream` (NULL = the null stream) and
 * never synchronises the host.  The calls hold no state across calls apart
 * from a per-device memory pool used by attn_jvp_fwd (and the calls below
 * given a NULL workspace) for its workspace: stream-ordered
 * hipMallocFromPoolAsync / hipFreeAsync, up to 2 GiB kept cached between
 * calls; concurrent calls from several threads or streams are safe.
 * attn_jvp_fwd_ws takes a caller-provided workspace instead, and
 * attn_jvp_fwd_noalloc a fixed buffer of the library's.
 *
 * Tuning.  The environment variable ATTN_JVP_TILE, read on every call, can
 * force the workgroup size of the bf16 kernels: 128 or 256 query rows for the
 * JVP (the default takes 128 when a work item has at most 16 key tiles), 256
 * or 512 for attn_fwd.  The results are the same bit for bit either way.
 *
 * Errors.  Argument errors are detected before anything is launched and leave
 * every output untouched:
 *   ATTN_JVP_EINVAL       a required pointer is NULL; B, H, Nq or Nk < 1;
 *                         `scale` is NaN or infinite; the workspace is NULL
 *                         or too small
 *   ATTN_JVP_EUNSUPPORTED d is not 64 or 128; one (b, h) slice of a tensor
 *                         reaches 2^31 bytes (counted as fp32: Nq*d*4 or
 *                         Nk*d*4), or one slice of the bf16 path's tile images
 *                         does (Nk beyond about 2 million at d = 128); B*H
 *                         exceeds 2^31 - 1
 *   ATTN_JVP_EALIGN       a tensor pointer is not 16-byte aligned (workspace:
 *                         256-byte aligned)
 *   ATTN_JVP_ELAUNCH      the HIP runtime rejected a launch or an allocation
 *                         (hipGetLastError); outputs are then unspecified
 * Device-side faults surface at the caller's next synchronisation.
 */
#ifndef ATTN_JVP_H
#define ATTN_JVP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ATTN_JVP_API __attribute__((visibility("default")))
#else
#define ATTN_JVP_API
#endif

#define ATTN_JVP_OK 0
#define ATTN_JVP_EINVAL (-1)
#define ATTN_JVP_EUNSUPPORTED (-2)
#define ATTN_JVP_EALIGN (-3)
#define ATTN_JVP_ELAUNCH (-4)

/* Output element types of attn_jvp_fwd_ex and attn_fwd. */
#define ATTN_JVP_OUT_F32 0
#define ATTN_JVP_OUT_BF16 1

/* Opaque HIP stream handle (hipStream_t). */
typedef struct ihipStream_t *attn_jvp_stream_t;

/*
 * Attention and its JVP, bf16 inputs, fp32 outputs (the operation above).
 *   q, k, v     primal inputs (bf16 bit patterns), layouts above
 *   tq, tk, tv  their tangents dQ, dK, dV (bf16), same layouts
 *   o, to       outputs O and dO, fp32 [B, H, Nq, d]
 *   lse         output row log-sum-exp, fp32 [B, H, Nq]; may be NULL (not written)
 *   B, H        batch and head counts; Nq, Nk query and key lengths (any >= 1;
 *               Nq != Nk is cross-attention); d = 64 or 128
 *   scale       softmax scale s, any finite value (typically 1/sqrt(d))
 *   stream      HIP stream for every launch
 * Allocates a workspace of attn_jvp_workspace_bytes(B, H, Nk, d) bytes from a
 * library-owned stream-ordered pool and frees it stream-ordered.
 * Returns ATTN_JVP_OK or an error code above.
 */
ATTN_JVP_API int attn_jvp_fwd(const void *q, const void *k, const void *v,
                 const void *tq, const void *tk, const void *tv,
                 float *o, float *to, float *lse,
                 int B, int H, int Nq, int Nk, int d, float scale,
                 attn_jvp_stream_t stream);

/*
 * attn_jvp_fwd for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * semantics and results (bit for bit) as attn_jvp_fwd; it calls no allocator.
 * The tile images live in a device buffer of ATTN_JVP_NOALLOC_BYTES that the
 * library holds on every GPU it runs on, from its first call there until the
 * process ends; a call whose images pass that size runs as consecutive
 * launches over groups of (b, h) slices that fit.  ATTN_JVP_EUNSUPPORTED if
 * the images of one slice do not fit (Nk beyond 131008 at d = 128, 262080
 * at d = 64); otherwise errors as attn_jvp_fwd.  Every call on one GPU uses
 * the same buffer: calls that may overlap on one GPU (other streams, other
 * threads) race and give wrong results; calls in one stream are ordered.
 */
#define ATTN_JVP_NOALLOC_BYTES ((size_t)128 << 20)
ATTN_JVP_API int attn_jvp_fwd_noalloc(const void *q, const void *k, const void *v,
                         const void *tq, const void *tk, const void *tv,
                         float *o, float *to, float *lse,
                         int B, int H, int Nq, int Nk, int d, float scale,
                         attn_jvp_stream_t stream);

/*
 * Bytes of workspace the bf16 path needs for these sizes: per (b, h), one
 * 64-key tile image per key tile, holding K and dK (bf16) and V^T and dV^T
 * (fp16, scaled by the slice's powers of two) as the sequence of matrix-core
 * operand fragments the fused kernel reads, laid out byte for byte as it holds
 * them in LDS (64 KiB per tile at d = 128, 32 KiB at d = 64), then a 2 KiB
 * header (the powers of two, the partial maxima they come from and the largest
 * key norms); 0 if a size is invalid.  Same operation as attn_jvp_fwd.
 */
ATTN_JVP_API size_t attn_jvp_workspace_bytes(int B, int H, int Nk, int d);

/*
 * attn_jvp_fwd with a caller-provided device workspace (256-byte aligned,
 * at least attn_jvp_workspace_bytes(B, H, Nk, d) bytes, not shared with a call
 * that may run concurrently).  Allocates nothing.  Same arguments, semantics and
 * errors as attn_jvp_fwd otherwise.
 */
ATTN_JVP_API int attn_jvp_fwd_ws(const void *q, const void *k, const void *v,
                    const void *tq, const void *tk, const void *tv,
                    float *o, float *to, float *lse,
                    int B, int H, int Nq, int Nk, int d, float scale,
                    void *workspace, size_t workspace_bytes,
                    attn_jvp_stream_t stream);

/*
 * The two phases of attn_jvp_fwd_ws, for callers that schedule, time or reuse
 * them separately (one packed workspace serves every call with the same K, V,
 * dK, dV, B, H, Nk and d, e.g. several query batches against one set of keys).
 *
 * attn_jvp_pack_kv converts k, v, tk, tv (bf16, [B, H, Nk, d]) to the tile
 * images described at attn_jvp_workspace_bytes and writes them to `workspace`
 * (256-byte aligned, at least attn_jvp_workspace_bytes(B, H, Nk, d) bytes),
 * overwriting all of it.  Errors as above (EINVAL for a NULL input or
 * workspace, or a short workspace).
 *
 * attn_jvp_fwd_packed computes O, dO and lse from q, tq and a workspace that
 * attn_jvp_pack_kv filled for the same B, H, Nk, d, ordered before this call
 * (same stream, or synchronised).  The workspace is only read.  Other
 * arguments and errors as attn_jvp_fwd.  Allocates nothing.
 */
ATTN_JVP_API int attn_jvp_pack_kv(const void *k, const void *v,
                     const void *tk, const void *tv,
                     int B, int H, int Nk, int d,
                     void *workspace, size_t workspace_bytes,
                     attn_jvp_stream_t stream);

ATTN_JVP_API int attn_jvp_fwd_packed(const void *q, const void *tq,
                        const void *workspace, size_t workspace_bytes,
                        float *o, float *to, float *lse,
                        int B, int H, int Nq, int Nk, int d, float scale,
                        attn_jvp_stream_t stream);

/*
 * Extended form of attn_jvp_fwd (same operation, same input layouts):
 *   tq, tk, tv   each may be NULL, meaning a zero tangent.  With tk = tv = NULL
 *                (frozen keys, e.g. the text keys of cross-attention) the
 *                products with dK and dV are left out: 4 of the 6 contractions.
 *   o, to        O and dO, [B, H, Nq, d], in fp32 (out_dtype ATTN_JVP_OUT_F32)
 *                or bf16 rounded to nearest even (ATTN_JVP_OUT_BF16); required
 *   lse          fp32 [B, H, Nq] or NULL
 *   tlse         the tangent of lse, mu_i = sum_j P_ij dS_ij, fp32 [B, H, Nq], or
 *                NULL.  With lse, O and dO it is the state that attn_jvp_merge
 *                combines across key subsets.
 *   workspace    NULL (a library-owned stream-ordered pool provides it) or a
 *                device buffer of at least attn_jvp_workspace_bytes(B, H, Nk, d)
 *                bytes, 256-byte aligned (then nothing is allocated)
 * Errors as attn_jvp_fwd; EINVAL also for an unknown out_dtype; EALIGN for a
 * non-NULL tangent not 16-byte aligned or tlse not 4-byte aligned.
 */
ATTN_JVP_API int attn_jvp_fwd_ex(const void *q, const void *k, const void *v,
                    const void *tq, const void *tk, const void *tv,
                    void *o, void *to, float *lse, float *tlse,
                    int B, int H, int Nq, int Nk, int d, float scale, int out_dtype,
                    void *workspace, size_t workspace_bytes,
                    attn_jvp_stream_t stream);

/*
 * Split-KV form of the same operation, for few query rows against many keys
 * (the merge of partial states that exporting the tangent of lse allows; the
 * rCM record in the Anthology of the SOTA, "Key takeaways", "JVP at
 * production scale", on the kernel composing with context parallelism): the
 * 64-key tiles are cut into contiguous ranges that run on separate
 * workgroups, each range's (lse, O, dO, mu) goes to the workspace, and the
 * merge of attn_jvp_merge combines them.
 *   q, k, v, tq, tk, tv, o, to, lse, tlse   as attn_jvp_fwd_ex (tangents may be
 *                NULL; tk = tv = NULL runs the frozen-key kernel); o, to fp32
 *   nsplit       number of ranges: 0 chooses one from the sizes (enough
 *                workgroups for two rounds on the chip, at least 4 tiles per
 *                range); a larger value than the tile count (or 1024) is
 *                clamped, and the count used is ceil(ntiles / ceil(ntiles /
 *                nsplit)).  With one range the result equals attn_jvp_fwd_ex's
 *                bit for bit.
 *   workspace    NULL (library pool) or at least
 *                attn_jvp_splitkv_workspace_bytes(B, H, Nq, Nk, d, nsplit)
 *                bytes, 256-byte aligned
 * Results differ from the unsplit pass by rounding only (sums regrouped).
 * Errors as attn_jvp_fwd_ex; EINVAL also for nsplit < 0.
 */
ATTN_JVP_API int attn_jvp_fwd_splitkv(const void *q, const void *k, const void *v,
                         const void *tq, const void *tk, const void *tv,
                         float *o, float *to, float *lse, float *tlse,
                         int B, int H, int Nq, int Nk, int d, float scale, int nsplit,
                         void *workspace, size_t workspace_bytes,
                         attn_jvp_stream_t stream);

/* Workspace bytes of attn_jvp_fwd_splitkv (tile images, then the partial
 * states when more than one range is used); 0 if a size is invalid.  The
 * range count is chosen per group of slices (a group whose partial O would
 * pass 2^31 bytes uses fewer ranges), and the groups of a call past 2^31
 * bytes per tensor reuse the workspace: it holds the larger group's need. */
ATTN_JVP_API size_t attn_jvp_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d,
                                                     int nsplit);

/*
 * attn_fwd (forward attention alone) with the key tiles cut into ranges as in
 * attn_jvp_fwd_splitkv, partial (lse, O) merged: for few query rows against
 * many keys.  o fp32 [B, H, Nq, d], lse fp32 [B, H, Nq] or NULL; nsplit and
 * the workspace as attn_jvp_fwd_splitkv (attn_jvp_splitkv_workspace_bytes
 * bytes suffice).  With one range the result equals attn_fwd's bit for bit.
 * Errors as attn_fwd; EINVAL also for nsplit < 0.
 */
ATTN_JVP_API int attn_fwd_splitkv(const void *q, const void *k, const void *v,
                     float *o, float *lse,
                     int B, int H, int Nq, int Nk, int d, float scale, int nsplit,
                     void *workspace, size_t workspace_bytes,
                     attn_jvp_stream_t stream);

/*
 * Forward attention alone (FlashAttention-2's output, without a tangent):
 * O = softmax(scale Q K^T) V and lse, bf16 inputs as in attn_jvp_fwd, O in fp32
 * or bf16 (out_dtype), lse fp32 or NULL.  The pass of attn_jvp_fwd with the
 * tangent left out (2 of the 6 contractions, 64 query rows per wave); its O and
 * lse equal attn_jvp_fwd's bit for bit.  Workspace and errors as
 * attn_jvp_fwd_ex.
 */
ATTN_JVP_API int attn_fwd(const void *q, const void *k, const void *v,
             void *o, float *lse,
             int B, int H, int Nq, int Nk, int d, float scale, int out_dtype,
             void *workspace, size_t workspace_bytes,
             attn_jvp_stream_t stream);

/*
 * Merge of P partial results of the same R query rows, each computed against
 * a disjoint subset of the keys (a key-split of one call, or the key shards
 * of a context-parallel layout).  fp32 device arrays, part-major:
 *   lse_parts [P][R], o_parts [P][R][d], to_parts [P][R][d], tlse_parts [P][R]
 *   lse [R], o [R][d], to [R][d], tlse [R]
 * with a_p = exp(lse_p - lse):  lse = log sum_p exp(lse_p),  O = sum_p a_p O_p,
 * tlse = sum_p a_p tlse_p,  dO = sum_p a_p (dO_p + tlse_p O_p) - tlse O.
 * to_parts, tlse_parts and to are either all given (the JVP state) or all NULL
 * (forward only; tlse must then be NULL too); lse may be NULL.  d = 64 or 128,
 * 1 <= P <= 1024; arrays of any size (rows past 2^31 bytes of one part's O run
 * as consecutive launches over chunks of rows).  A row whose parts all have
 * lse = -inf yields NaN.  Errors: EINVAL (NULL inputs, inconsistent tangent
 * arguments, P or R < 1), EUNSUPPORTED (d or P), EALIGN (16-byte for o/to
 * arrays, 4-byte for lse/tlse arrays), ELAUNCH.  Allocates nothing.
 */
ATTN_JVP_API int attn_jvp_merge(const float *lse_parts, const float *o_parts,
                   const float *to_parts, const float *tlse_parts,
                   int P, int R, int d,
                   float *lse, float *o, float *to, float *tlse,
                   attn_jvp_stream_t stream);

/*
 * Backward pass of the same attention (FlashAttention-2's reverse mode): the
 * gradients of a loss L with respect to Q, K and V, given gO = dL/dO.  Per
 * (b, h), with P = softmax(scale Q K^T) = exp(scale Q K^T - lse):
 *   gV = P^T gO,  gS = P * (gO V^T - D),  D_i = <gO_i, O_i>,
 *   gQ = scale gS K,  gK = scale gS^T Q.
 *   q, k, v, go  bf16 [B, H, Nq|Nk, d] (go like q)
 *   o, lse       the forward's fp32 O [B, H, Nq, d] and lse [B, H, Nq] for the
 *                same q, k, v, scale (attn_fwd or attn_jvp_fwd output)
 *   gq, gk, gv   fp32 outputs, [B, H, Nq, d], [B, H, Nk, d], [B, H, Nk, d]
 *   workspace    NULL (library pool) or at least attn_bwd_workspace_bytes(B, H,
 *                Nq, Nk, d) bytes, 256-byte aligned (then nothing is allocated)
 * bf16 products with fp32 accumulation; P and the softmax gradient gS are
 * rounded to fp16 for the products with gO^T, Q^T and K^T.  Errors as
 * attn_jvp_fwd (EINVAL: a NULL pointer, sizes < 1, bad scale, short
 * workspace; EUNSUPPORTED: d, B*H, or one (b, h) slice of a tensor or of the
 * workspace's tile images reaching 2^31 bytes; EALIGN: 16-byte tensors, 4-byte
 * lse, 256-byte workspace).  Calls past 2^31 bytes per tensor run in groups of
 * slices that reuse the workspace in stream order, as for split-KV.
 */
ATTN_JVP_API int attn_bwd(const void *q, const void *k, const void *v,
             const float *o, const void *go, const float *lse,
             float *gq, float *gk, float *gv,
             int B, int H, int Nq, int Nk, int d, float scale,
             void *workspace, size_t workspace_bytes,
             attn_jvp_stream_t stream);

/* Workspace bytes of attn_bwd (tile images of Q, gO and of K, V); 0 if a size
 * is invalid. */
ATTN_JVP_API size_t attn_bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d);

/*
 * The same operation with fp32 inputs and fp32 arithmetic throughout (the
 * precision reference path).  Same layouts, arguments and errors; needs no
 * workspace and allocates nothing.
 */
ATTN_JVP_API int attn_jvp_fwd_f32(const float *q, const float *k, const float *v,
                     const float *tq, const float *tk, const float *tv,
                     float *o, float *to, float *lse,
                     int B, int H, int Nq, int Nk, int d, float scale,
                     attn_jvp_stream_t stream);

/* Static, human-readable name of a status code (never NULL). */
ATTN_JVP_API const char *attn_jvp_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_JVP_H */
