/*
 * mhc.h -- C ABI of libmhc: the mHC (manifold-constrained hyper-connections)
 * residual-stream forward on one AMD Instinct MI355X (gfx950).
 *
 * The method is the one stated in section 2 of the blog page
 * "mHC 算法分析 & cutile 高效实现" (edward-lyz, 2026-02-10), cited below as
 * [mHC-cutile].  Three calls cover the forward of one mHC layer:
 *
 *   mhc_coeffs    steps (1)-(3): logits = X_t . phi and r = RMS(X_t) in one
 *                 pass over X_t, then the alpha/r + bias correction, the
 *                 sigmoid / 2*sigmoid gates and 20 Sinkhorn-Knopp iterations;
 *   mhc_pre       step (4a): F_pre = sum_i H_pre[i] X_t[i]   (n streams -> 1);
 *   mhc_post_res  step (4b): X_next[i] = sum_j H_res[i,j] X_t[j] + H_post[i] F_out.
 *
 * Between mhc_pre and mhc_post_res the caller runs its own layer F
 * (attention / FFN) to turn F_pre into F_out; that layer is not part of mHC.
 * mhc_post_res_coeffs fuses a layer's apply with the next layer's
 * coefficients (one pass over the residual stream instead of two).
 *
 * Conventions shared by every call
 * --------------------------------
 *  B   number of rows (tokens = batch x sequence), B >= 0;
 *  n   expansion rate (number of residual streams), one of 1, 2, 4, 8;
 *  C   hidden size, C >= 8 and C % 8 == 0;
 *  N   = n*n + 2n coefficients per row, K = n*C.
 *
 *  bf16 tensors are raw bfloat16 bit patterns (uint16), row-major.  X_t is
 *  [B, n*C] stream-major: stream j occupies columns [j*C, (j+1)*C) of a row
 *  ([mHC-cutile] sections 2 and 5.4).  A coefficient row is laid out
 *  [pre (n) | post (n) | res (n*n, row-major (i, j))], the column order of the
 *  single product in [mHC-cutile] section 2.1.
 *
 *  All tensor pointers are DEVICE pointers owned by the caller.  The library
 *  allocates and frees nothing and keeps no pointer after a call returns.
 *  bf16 tensors and the workspace must be 16-byte aligned; fp32 tensors
 *  4-byte aligned.  `stream` is a hipStream_t (NULL = the null stream).
 *
 *  Every call only enqueues work on `stream` and returns; it never
 *  synchronises the host or the device.  Inputs must stay valid until the
 *  stream has passed the call.  Calls are stateless and thread-safe.
 *
 *  Errors: every call returns an mhc_status value and never aborts, throws or
 *  prints.  Arguments are checked on the host before anything is launched:
 *    - a required pointer is NULL, B < 0, n < 1 or C < 1     -> MHC_ERR_INVALID_ARG
 *    - an output overlaps an input or another output        -> MHC_ERR_INVALID_ARG
 *    - n not in {1,2,4,8}, C % 8 != 0, misaligned pointer   -> MHC_ERR_UNSUPPORTED
 *    - workspace smaller than mhc_coeffs_workspace_size()    -> MHC_ERR_WORKSPACE
 *    - the HIP runtime reports a launch error                -> MHC_ERR_HIP
 *  B == 0 is valid and launches nothing.  MHC_ERR_INCOMPLETE is returned only
 *  by mhc_post_res_coeffs_pre_check and mhc_coeffs_pre_check (below).  Faults during asynchronous
 *  execution surface at the caller's next synchronisation, as in HIP.
 */
#ifndef MHC_H
#define MHC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sinkhorn-Knopp (row, column) normalisation pairs: [mHC-cutile] section 2.4
 * gives about 20; its kernels in sections 4.3 and 5.3 fix exactly 20. */
#define MHC_SINKHORN_ITERS 20

enum mhc_status {
  MHC_OK = 0,
  MHC_ERR_INVALID_ARG = 1,
  MHC_ERR_UNSUPPORTED = 2,
  MHC_ERR_WORKSPACE = 3,
  MHC_ERR_HIP = 4,
  MHC_ERR_INCOMPLETE = 5
};

/* Human-readable name of a status code (static storage; never NULL). */
const char *mhc_status_string(int status);

/* Bytes of device workspace mhc_coeffs needs for (B, n, C): the split-K
 * partial sums, fp32 [S, B, N+1], plus (up to 256 rows) one 8-byte arrival
 * flag per 16-row tile and K-slice, or (above) a packed copy of phi.  Returns
 * 0 for B == 0 or for arguments mhc_coeffs would reject.  Pure host
 * function. */
size_t mhc_coeffs_workspace_size(int64_t B, int32_t n, int64_t C);

/* Number S of K-slices mhc_coeffs splits the reduction over K = n*C into for
 * (B, n, C); 0 for arguments mhc_coeffs would reject.  Pure host function,
 * for introspection. */
int32_t mhc_coeffs_split_k(int64_t B, int32_t n, int64_t C);

/* Steps (1)-(3) of the forward.
 *
 * [mHC-cutile] section 2.1: logits = X_t . phi (one product for all N
 * columns); section 2.2: r = sqrt(sum(X_t^2) / (n C)) per row, no epsilon;
 * section 2.3: h = alpha_x * logit / r + b_x; section 2.4: H_pre = sigmoid(h),
 * H_post = 2 sigmoid(h), H_res = Sinkhorn-Knopp(exp(h)) with 20 row-then-
 * column normalisations.  [mHC-cutile] sections 3.1 and 5.1-5.3 motivate the
 * fusion: one pass over X_t gives both the product and the sum of squares
 * (applying 1/r after the product is the row-scaling identity of section 2 of
 * "Towards Free Normalization: Fusing Normalization into GEMM and Attention
 * Kernels").
 *
 *   X_t       in  bf16 [B, n*C]
 *   phi       in  bf16 [n*C, N], row-major
 *   alpha_*   in  host fp32 scalars
 *   b_pre     in  fp32 [n];  b_post in fp32 [n];  b_res in fp32 [n*n] row-major
 *   logits    out fp32 [B, N]  raw X_t . phi
 *   r         out fp32 [B]
 *   H         out fp32 [B, N]  [H_pre | H_post | H_res]
 *   workspace scratch, >= mhc_coeffs_workspace_size(B, n, C) bytes; its
 *             contents on entry are ignored and on exit undefined.
 *
 * The result is deterministic: the split-K partials are combined in a fixed
 * order.  Up to 256 rows the call is a single kernel (the decode sizes of
 * [mHC-cutile] section 3.2, where launches dominate): the K-slices of each
 * 16-row tile publish their partials and arrival flags in the workspace, and
 * whichever slice finds all flags set adds the partials in slice order and
 * finishes the tile.  The flags carry a per-call tag, so the workspace needs
 * no initialisation in either case. */
int mhc_coeffs(int64_t B, int32_t n, int64_t C,
               const void *X_t, const void *phi,
               float alpha_pre, float alpha_post, float alpha_res,
               const float *b_pre, const float *b_post, const float *b_res,
               float *logits, float *r, float *H,
               void *workspace, size_t workspace_bytes, void *stream);

/* Step (4a), [mHC-cutile] section 2.5: F_pre[b, c] = sum_i H_pre[b, i] *
 * X_t[b, i*C + c], accumulated in fp32 and rounded to bf16 (nearest even).
 *
 *   X_t    in  bf16 [B, n*C]
 *   H      in  fp32 [B, N] (only the pre block is read)
 *   F_pre  out bf16 [B, C] */
int mhc_pre(int64_t B, int32_t n, int64_t C, const void *X_t, const float *H,
            void *F_pre, void *stream);

/* Step (4b), [mHC-cutile] sections 2.5 and 3.4: X_next[b, i*C + c] =
 * sum_j H_res[b, i, j] * X_t[b, j*C + c] + H_post[b, i] * F_out[b, c],
 * accumulated in fp32 and rounded to bf16 (nearest even).  X_t is read once
 * and X_next written once.
 *
 *   X_t     in  bf16 [B, n*C]
 *   F_out   in  bf16 [B, C]
 *   H       in  fp32 [B, N] (the post and res blocks are read)
 *   X_next  out bf16 [B, n*C]; must not overlap X_t */
int mhc_post_res(int64_t B, int32_t n, int64_t C, const void *X_t,
                 const void *F_out, const float *H, void *X_next, void *stream);

/* Step (4b) of this layer fused with steps (1)-(3) of the next one.
 *
 * The apply of [mHC-cutile] sections 2.5 and 3.4 writes X_next, which is the
 * next layer's input X_t; section 2.1 then begins the next layer with the
 * product X_next . phi_next (and section 2.2 with the row sums of X_next^2).
 * This call performs both in one pass over the residual stream, so X_next is
 * written once and never read back for the next layer's coefficients:
 *
 *   X_next       = exactly what mhc_post_res(X_t, F_out, H) writes (bitwise);
 *   logits_next, r_next, H_next
 *                = what mhc_coeffs(X_next, phi_next, alpha_*, b_*) computes,
 *                  up to fp32 summation order (deterministic, no atomics).
 *
 * A model runs mhc_coeffs once for its first layer and then, per layer,
 * mhc_pre, its layer F, and this call.  Arguments as in mhc_post_res
 * (X_t, F_out, H, X_next) and mhc_coeffs (phi_next, alpha_*, b_*, logits_next,
 * r_next, H_next, workspace).  Additionally requires C % 32 == 0
 * (else MHC_ERR_UNSUPPORTED); the workspace must hold
 * mhc_post_res_coeffs_workspace_size(B, n, C) bytes.  At n = 8 (B above
 * 256, C <= 4096) the pass splits each row into C/128 slices of 128 channels
 * of all eight streams, so the workspace holds fp32 partials [C/128, B, 81]
 * (85 MB at B = 8192, C = 4096). */
size_t mhc_post_res_coeffs_workspace_size(int64_t B, int32_t n, int64_t C);

int mhc_post_res_coeffs(int64_t B, int32_t n, int64_t C,
                        const void *X_t, const void *F_out, const float *H, void *X_next,
                        const void *phi_next,
                        float alpha_pre, float alpha_post, float alpha_res,
                        const float *b_pre, const float *b_post, const float *b_res,
                        float *logits_next, float *r_next, float *H_next,
                        void *workspace, size_t workspace_bytes, void *stream);

/* The whole per-layer mHC forward after the layer F, in one pass: step (4b)
 * of this layer, then steps (1)-(3) and step (4a) of the next.
 *
 * [mHC-cutile] section 2.5 (first step) forms the next layer's input
 * F_pre = sum_i H_pre[i] X_next[i] once the next layer's H_pre is known
 * (sections 2.1-2.4).  This call returns everything mhc_post_res_coeffs
 * returns and, in addition,
 *
 *   F_pre_next   out bf16 [B, C] = exactly what mhc_pre(X_next, H_next) writes
 *                (bitwise).
 *
 * A model runs mhc_coeffs_pre (or mhc_coeffs and mhc_pre) once for its first
 * layer and then, per layer, its layer F and this call: the residual stream
 * is read once and written once per layer (X_t and F_out in, X_next and
 * F_pre_next out).
 *
 * Where the shape allows (n <= 4, B above 256, C % 32 == 0 and at most 16
 * 512-channel steps per row, i.e. C <= 8192) this runs as one persistent
 * pass whose workgroups exchange each row's partial sums through the
 * workspace; mhc_post_res_coeffs_pre_one_pass() reports whether a shape takes
 * that route.  The workgroups of a round wait for each other, so the call
 * sizes that pass's grid to what can be resident at once -- the occupancy
 * the HIP runtime reports for the kernel (one workgroup per compute unit)
 * times the compute units `stream` may use (its CU mask) -- and runs the two
 * calls below instead when not even one row's slices fit together.  It
 * cannot see kernels that other streams or processes run at the same time:
 * if they hold compute units so long that a wait for another workgroup
 * cannot complete within about a second, the wait gives up, writes NaN to the
 * affected F_pre_next vectors and sets a word in the workspace, which
 * mhc_post_res_coeffs_pre_check reads back.  Where all of a row's channels
 * fit one 1024-channel slice (bf16, n <= 4, B <= 256, n*C <= 1024) it runs
 * as one kernel with one workgroup per 16 rows: no workgroup waits for
 * another and the workspace is not touched (its size is still required), and
 * mhc_post_res_coeffs_pre_one_pass() reports 1 for these shapes too.  Other
 * shapes run mhc_post_res_coeffs followed by mhc_pre on X_next, with the same
 * results; at n = 8 that is the default (a one pass at n = 8 exists, for
 * C <= 4096, behind the MHC_PASS8_PRE tuning key below: measured slower).
 *
 * Arguments as mhc_post_res_coeffs, plus F_pre_next (16-byte aligned, must
 * not overlap any other argument).  The workspace must hold
 * mhc_post_res_coeffs_pre_workspace_size(B, n, C) bytes; its contents on
 * entry do not matter. */
size_t mhc_post_res_coeffs_pre_workspace_size(int64_t B, int32_t n, int64_t C);

int mhc_post_res_coeffs_pre(int64_t B, int32_t n, int64_t C,
                            const void *X_t, const void *F_out, const float *H, void *X_next,
                            const void *phi_next,
                            float alpha_pre, float alpha_post, float alpha_res,
                            const float *b_pre, const float *b_post, const float *b_res,
                            float *logits_next, float *r_next, float *H_next, void *F_pre_next,
                            void *workspace, size_t workspace_bytes, void *stream);

/* 1 if mhc_post_res_coeffs_pre runs this shape as one pass (the persistent
 * pass, or the single-slice kernel at small shapes), 0 if it runs the two
 * calls (or the shape is invalid).  (A stream whose CU mask leaves too few
 * compute units makes the persistent pass's shapes take the two calls even
 * where this returns 1.) */
int32_t mhc_post_res_coeffs_pre_one_pass(int64_t B, int32_t n, int64_t C);

/* Whether the last mhc_post_res_coeffs_pre (fp8 == 0) or
 * mhc_post_res_coeffs_pre_fp8 (fp8 != 0) call of shape (B, n, C) that used
 * `workspace` completed every wait of its one-pass route.  Synchronises
 * `stream` (the stream of that call) and reads one word of the workspace;
 * the workspace must still be the one the call used, not yet reused.
 * workspace == NULL reads the word of mhc_post_res_coeffs_pre_noalloc's
 * array on the current device instead (fp8 must then be 0).
 * Returns MHC_OK when no wait gave up (always for shapes that run the two
 * calls), MHC_ERR_INCOMPLETE when one did (F_pre_next then holds NaN -- the
 * E4M3 code 0x7F in the fp8 call -- in the vectors of the rows it gave up
 * on; X_next, logits_next, r_next and H_next are still complete), and the
 * usual argument errors and MHC_ERR_HIP otherwise. */
int mhc_post_res_coeffs_pre_check(int64_t B, int32_t n, int64_t C, int32_t fp8,
                                  const void *workspace, size_t workspace_bytes, void *stream);

/* mhc_post_res_coeffs_pre for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call, results and routes, without the workspace
 * argument.  Its workspace is a device array inside the library, of
 * MHC_NOALLOC_SCRATCH_BYTES (32 MiB: the large workload n = 4, C = 7168,
 * B = 16384 needs about 28.4 MB), one per GPU the library runs on, held until
 * the process ends.  Shapes whose workspace (as
 * mhc_post_res_coeffs_pre_workspace_size reports it) exceeds that return
 * MHC_ERR_WORKSPACE before anything is launched, except at n = 8: where the
 * n = 8 pass's partials would not fit (C/128 slices x B x 81 fp32, above
 * B = 3236 at C = 4096) the call takes the apply and split-K product route,
 * whose workspace does, so the coefficients may differ from the workspace
 * call's in fp32 summation order (X_next and F_pre_next bitwise as always
 * against mhc_post_res and mhc_pre).  The call allocates nothing:
 * the first call on a device looks up the array's device address once.
 * Every call on a GPU shares that GPU's array, so calls that overlap in time
 * on one GPU (on different streams, or from different threads) race and must
 * be ordered by the caller; calls on one stream are ordered by the stream.
 * The array keeps whatever the last call left; each call clears what must
 * start at zero with its own kernels.  The give-up word of the one-pass route
 * is in the array too: mhc_post_res_coeffs_pre_check with workspace NULL
 * reads it. */
#define MHC_NOALLOC_SCRATCH_BYTES (32u << 20)

int mhc_post_res_coeffs_pre_noalloc(int64_t B, int32_t n, int64_t C,
                                    const void *X_t, const void *F_out, const float *H,
                                    void *X_next, const void *phi_next,
                                    float alpha_pre, float alpha_post, float alpha_res,
                                    const float *b_pre, const float *b_post, const float *b_res,
                                    float *logits_next, float *r_next, float *H_next,
                                    void *F_pre_next, void *stream);

/* Steps (1)-(3) and step (4a) of one layer in one pass over X_t: the first
 * layer's counterpart of mhc_post_res_coeffs_pre, for a stream that no apply
 * produced (the layer-0 X_t built from the embeddings).
 *
 * [mHC-cutile] section 3.1 forms the product and the sum of squares in one
 * pass over X_t, and section 2.5 (first step) needs F_pre = sum_i H_pre[i]
 * X_t[i] once H_pre (sections 2.1-2.4) is known.  This call returns
 *
 *   logits, r, H = what mhc_coeffs(X_t, phi, alpha_*, b_*) computes, up to
 *                  fp32 summation order (deterministic, no atomics);
 *   F_pre    out bf16 [B, C] = exactly what mhc_pre(X_t, H) writes with the
 *                  H this call returns (bitwise).
 *
 * Arguments as mhc_coeffs plus F_pre (16-byte aligned, must not overlap any
 * other argument).  The workspace must hold mhc_coeffs_pre_workspace_size(B,
 * n, C) bytes; its contents on entry do not matter.  Where
 * mhc_post_res_coeffs_pre takes its one pass (and C % 32 == 0),
 * mhc_coeffs_pre_one_pass() returns 1 and the call is the same persistent
 * pass without the apply: X_t is read once, nothing is written back to it,
 * and the residency rules, the give-up behaviour (F_pre NaN in the rows a
 * wait gave up on; logits, r and H still complete) and the give-up word
 * (read with mhc_coeffs_pre_check) are those of mhc_post_res_coeffs_pre.
 * Where mhc_post_res_coeffs_pre takes its single-slice kernel (bf16, n <= 4,
 * B <= 256, n*C <= 1024; here also for C % 32 != 0, C % 8 == 0) this call
 * takes the same kernel without the apply.  Other shapes run mhc_coeffs
 * followed by mhc_pre, with the same results. */
size_t mhc_coeffs_pre_workspace_size(int64_t B, int32_t n, int64_t C);

int mhc_coeffs_pre(int64_t B, int32_t n, int64_t C,
                   const void *X_t, const void *phi,
                   float alpha_pre, float alpha_post, float alpha_res,
                   const float *b_pre, const float *b_post, const float *b_res,
                   float *logits, float *r, float *H, void *F_pre,
                   void *workspace, size_t workspace_bytes, void *stream);

/* 1 if mhc_coeffs_pre runs this shape as one pass, 0 otherwise (as
 * mhc_post_res_coeffs_pre_one_pass, which it equals for C % 32 == 0). */
int32_t mhc_coeffs_pre_one_pass(int64_t B, int32_t n, int64_t C);

/* Whether the last mhc_coeffs_pre (fp8 == 0) or mhc_coeffs_pre_fp8 (fp8 != 0)
 * call of shape (B, n, C) that used `workspace` completed every wait of its
 * one-pass route; as mhc_post_res_coeffs_pre_check (synchronises `stream`,
 * reads one word; workspace must not be NULL).  MHC_OK when no wait gave up
 * (always for shapes that run the two calls), MHC_ERR_INCOMPLETE when one did. */
int mhc_coeffs_pre_check(int64_t B, int32_t n, int64_t C, int32_t fp8,
                         const void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * FP8 residual-stream variant.
 *
 * [mHC-cutile] runs its first benchmark (the performance section after its
 * section 4 kernels) with every tensor in torch.float8_e4m3fn.  These calls
 * are the three above (and the fused call) with the residual-stream tensors
 * X_t, F_out, F_pre and X_next in FP8 E4M3 -- the OCP "fn" encoding: 1 sign,
 * 4 exponent (bias 7) and 3 mantissa bits, subnormals, no infinities, NaN =
 * S.1111.111, largest finite value 448 -- stored unscaled, one byte per
 * element, same layouts as the bf16 calls.  phi stays bf16 and H, logits, r
 * stay fp32.
 *
 * Readings (the page gives no conversion rules): values are used as they are
 * (no scale factors, as in the page's benchmark); inputs are widened exactly;
 * arithmetic is fp32 as in the bf16 calls, except that at n = 4 the post/res
 * mix of X_next runs on the matrix core with each coefficient carried as two
 * bf16 parts (to 2^-18 relative; products exact, fp32 sums), which can move
 * an E4M3 result only where the exact value lies within about 2^-17 of its
 * terms' magnitude from a rounding midpoint; F_pre and X_next are rounded
 * once to E4M3, to nearest even, saturating at +-448 (torch's own cast
 * returns NaN past the range); a NaN (from a NaN input) stays NaN, as code
 * 0x7F or 0xFF.  The product widens the E4M3 X exactly to bf16 for the
 * matrix core, so logits, r and H carry the bf16 calls' accuracy.
 *
 * Arguments, ownership, errors and workspace rules are those of the bf16
 * calls, with E4M3 in place of bf16 and the additional requirement
 * C % 16 == 0 (16-byte vectors of 16 elements), else MHC_ERR_UNSUPPORTED.
 * Workspace sizes come from the *_fp8_workspace_size functions.
 * ------------------------------------------------------------------------ */

size_t mhc_coeffs_fp8_workspace_size(int64_t B, int32_t n, int64_t C);

/* Steps (1)-(3) on an E4M3 X_t [B, n*C]; as mhc_coeffs otherwise (up to 256
 * rows one kernel, above that the split-K product with X staged through LDS,
 * then the combine kernel). */
int mhc_coeffs_fp8(int64_t B, int32_t n, int64_t C,
                   const void *X_t, const void *phi,
                   float alpha_pre, float alpha_post, float alpha_res,
                   const float *b_pre, const float *b_post, const float *b_res,
                   float *logits, float *r, float *H,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Step (4a): F_pre (E4M3 [B, C]) = sum_i H_pre[b, i] * X_t[b, i*C + c]. */
int mhc_pre_fp8(int64_t B, int32_t n, int64_t C, const void *X_t, const float *H,
                void *F_pre, void *stream);

/* Step (4b): X_next (E4M3 [B, n*C]) from X_t and F_out (both E4M3). */
int mhc_post_res_fp8(int64_t B, int32_t n, int64_t C, const void *X_t,
                     const void *F_out, const float *H, void *X_next, void *stream);

/* mhc_post_res_coeffs on the E4M3 residual stream: X_next is bitwise what
 * mhc_post_res_fp8 writes; logits_next, r_next, H_next are what
 * mhc_coeffs_fp8(X_next, ...) computes, up to fp32 summation order.
 * Requires C % 32 == 0. */
size_t mhc_post_res_coeffs_fp8_workspace_size(int64_t B, int32_t n, int64_t C);

int mhc_post_res_coeffs_fp8(int64_t B, int32_t n, int64_t C,
                            const void *X_t, const void *F_out, const float *H, void *X_next,
                            const void *phi_next,
                            float alpha_pre, float alpha_post, float alpha_res,
                            const float *b_pre, const float *b_post, const float *b_res,
                            float *logits_next, float *r_next, float *H_next,
                            void *workspace, size_t workspace_bytes, void *stream);

/* mhc_post_res_coeffs_pre on the E4M3 residual stream ([mHC-cutile] section
 * 2.5 for F_pre, sections 2.1-2.4 for the coefficients it needs): everything
 * mhc_post_res_coeffs_fp8 returns, plus
 *
 *   F_pre_next   out E4M3 [B, C] = exactly what mhc_pre_fp8(X_next, H_next)
 *                writes (bitwise).
 *
 * Route, residency handling and give-up behaviour (NaN, here the E4M3 code
 * 0x7F, in the affected F_pre_next bytes; mhc_post_res_coeffs_pre_check with
 * fp8 = 1 reads it back) as for mhc_post_res_coeffs_pre; the
 * one-pass route also needs the fused E4M3 route (the default at n <= 4;
 * MHC_FUSED_FP8=0 turns it off), else the call runs mhc_post_res_coeffs_fp8
 * followed by mhc_pre_fp8 on X_next, with the same results.  Requires
 * C % 32 == 0; F_pre_next 16-byte aligned and not overlapping any other
 * argument; the workspace must hold mhc_post_res_coeffs_pre_fp8_workspace_size
 * bytes. */
size_t mhc_post_res_coeffs_pre_fp8_workspace_size(int64_t B, int32_t n, int64_t C);

int mhc_post_res_coeffs_pre_fp8(int64_t B, int32_t n, int64_t C,
                                const void *X_t, const void *F_out, const float *H,
                                void *X_next, const void *phi_next,
                                float alpha_pre, float alpha_post, float alpha_res,
                                const float *b_pre, const float *b_post, const float *b_res,
                                float *logits_next, float *r_next, float *H_next,
                                void *F_pre_next, void *workspace, size_t workspace_bytes,
                                void *stream);

/* 1 if mhc_post_res_coeffs_pre_fp8 runs this shape as one pass, else 0. */
int32_t mhc_post_res_coeffs_pre_fp8_one_pass(int64_t B, int32_t n, int64_t C);

/* mhc_coeffs_pre on an E4M3 X_t: what mhc_coeffs_fp8 returns, plus
 *
 *   F_pre    out E4M3 [B, C] = exactly what mhc_pre_fp8(X_t, H) writes with
 *            the H this call returns (bitwise).
 *
 * One pass where mhc_post_res_coeffs_pre_fp8 takes one (and C % 32 == 0),
 * else mhc_coeffs_fp8 followed by mhc_pre_fp8; give-up behaviour as
 * mhc_post_res_coeffs_pre_fp8 (mhc_coeffs_pre_check with fp8 = 1).  Requires
 * C % 16 == 0; the workspace must hold mhc_coeffs_pre_fp8_workspace_size
 * bytes. */
size_t mhc_coeffs_pre_fp8_workspace_size(int64_t B, int32_t n, int64_t C);

int mhc_coeffs_pre_fp8(int64_t B, int32_t n, int64_t C,
                       const void *X_t, const void *phi,
                       float alpha_pre, float alpha_post, float alpha_res,
                       const float *b_pre, const float *b_post, const float *b_res,
                       float *logits, float *r, float *H, void *F_pre,
                       void *workspace, size_t workspace_bytes, void *stream);

/* 1 if mhc_coeffs_pre_fp8 runs this shape as one pass, else 0. */
int32_t mhc_coeffs_pre_fp8_one_pass(int64_t B, int32_t n, int64_t C);

/* ------------------------------------------------------------------------
 * fp32 phi variant.
 *
 * The tuned benchmark of [mHC-cutile] section 5 keeps X in bf16, phi (its W)
 * in fp32 and every other input in fp32, and the product of section 5.1
 * multiplies in TF32 when either operand is fp32.  These calls take phi as
 * fp32 [n*C, N] row-major (16-byte aligned) and compute the product at
 * higher precision than TF32: phi is split into phi_hi = bf16(phi) and
 * phi_lo = bf16(phi - phi_hi), which together are within 2^-16 of phi
 * (relative), and the product is X . phi_hi + X . phi_lo accumulated in fp32
 * (bf16 X times either part is exact in fp32).  Everything else -- arguments,
 * outputs, ownership, errors, determinism -- is as for mhc_coeffs and
 * mhc_post_res_coeffs with a bf16 residual stream.  Workspace sizes come from
 * the *_phi32_workspace_size functions.  The product runs in the one-launch
 * small-B kernel up to 256 rows, otherwise in the split-K product staged
 * through LDS; mhc_post_res_coeffs_phi32 is then the apply followed by that
 * product on X_next (the fused kernel takes bf16 phi only).
 * ------------------------------------------------------------------------ */

size_t mhc_coeffs_phi32_workspace_size(int64_t B, int32_t n, int64_t C);

int mhc_coeffs_phi32(int64_t B, int32_t n, int64_t C,
                     const void *X_t, const float *phi,
                     float alpha_pre, float alpha_post, float alpha_res,
                     const float *b_pre, const float *b_post, const float *b_res,
                     float *logits, float *r, float *H,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Requires C % 32 == 0, as mhc_post_res_coeffs. */
size_t mhc_post_res_coeffs_phi32_workspace_size(int64_t B, int32_t n, int64_t C);

int mhc_post_res_coeffs_phi32(int64_t B, int32_t n, int64_t C,
                              const void *X_t, const void *F_out, const float *H, void *X_next,
                              const float *phi_next,
                              float alpha_pre, float alpha_post, float alpha_res,
                              const float *b_pre, const float *b_post, const float *b_res,
                              float *logits_next, float *r_next, float *H_next,
                              void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Lazy Pre-Norm GEMM (a second workload on the same machinery).
 *
 * Section 2 of the page "Towards Free Normalization: Fusing Normalization
 * into GEMM and Attention Kernels" ([FreeNorm]) defines
 *     C = rmsnorm(A) @ B,  rmsnorm(A) = A * rstd[:, None],
 *     rstd = rsqrt(sum(A^2, dim=-1) / K + eps)   (eps = 1e-5 on the page,
 * no element-wise affine weight), and computes it lazily: the product runs on
 * the raw A, the row sums of squares accumulate in the same k-loop, and each
 * output row is scaled by rstd at the end (a row scaling commutes with the
 * product).  [mHC-cutile] section 2.2's r is the same statistic without eps.
 *
 *   A     in  bf16 [M, K] row-major
 *   W     in  bf16 [N, K] row-major: B passed as its transpose, the layout of a
 *             linear layer's weight (both operands then have K contiguous)
 *   eps   host fp32 (1e-5 in [FreeNorm])
 *   C     out bf16 [M, N] row-major, fp32 accumulation, one round-to-nearest-
 *             even at the end
 *   rstd  out fp32 [M], or NULL if not wanted
 *
 * Requires K % 8 == 0 and N % 8 == 0 (16-byte rows), K <= 2^22 and
 * M * N, M * K, N * K <= 2^40, else MHC_ERR_UNSUPPORTED; M == 0 launches
 * nothing; N < 1 or K < 1 is MHC_ERR_INVALID_ARG.  No workspace.  Other
 * rules as for the calls above. */
int mhc_lazy_prenorm_gemm(int64_t M, int64_t N, int64_t K, const void *A, const void *W,
                          float eps, void *C, float *rstd, void *stream);

/* ------------------------------------------------------------------------
 * Testing and tuning.
 *
 * Every call above picks its kernels and launch shapes by the sizes of the
 * problem alone (the choices measured fastest on MI355X); the library reads
 * no environment variable.  These functions override the choices for tests
 * and tuning runs, process-wide, e.g. to run the register-path product or
 * the small-B kernel at any B.  Keys (value < 0 restores the default):
 *   MHC_SMALL_MAX_B  rows up to which the one-launch small-B coefficient
 *                    kernel runs (0: never)
 *   MHC_GEMM_ALGO    0: register-path product; 2: persistent product
 *                    kernel; 3: the n = 8 pass (product only)
 *   MHC_SPLIT_K, MHC_GEMM_WGS, MHC_GEMM_MB, MHC_GEMM_WAVES   split-K
 *                    product shape (K-slices, target workgroups, 16-row
 *                    blocks per wave, 4 or 8 waves per workgroup)
 *   MHC_GEMM_KC, MHC_GEMM_STAGES   128 with 5 or 6: the bf16 split-K product
 *                    at n <= 4 in 128-k chunks with a deeper ring
 *   MHC_GEMM_XREG    2: the bf16 split-K product (n = 4, 8) with X and phi
 *                    loaded through registers
 *   MHC_FUSED_N8     0: n = 8 as the apply and the split-K product; > 0:
 *                    the fused kernel (otherwise the n = 8 pass up to
 *                    C = 4096)
 *   MHC_FUSED_FP8    0: E4M3 fused call as apply + product; > 0: fused kernel
 *   MHC_FUSED_FIXED  0 / 1: the fused kernel's fixed-slice layout off / on
 *   MHC_FUSED_SPU, MHC_FUSED_WGS   fused kernel's steps per unit, grid cap
 *   MHC_FUSED_PRE    0: mhc_post_res_coeffs_pre(_fp8) as two calls
 *   MHC_APPLY_SMALL  0: small-B bf16 mhc_post_res_coeffs as the apply
 *                    kernel, then the small-B coefficient kernel
 *   MHC_LPN_ALGO     1: the four-wave Lazy Pre-Norm GEMM kernel
 *   MHC_PASS8_SETS   1 or 2: register sets of loads in flight per wave of
 *                    the n = 8 one pass (mhc_post_res_coeffs_pre,
 *                    mhc_coeffs_pre)
 *   MHC_PASS8_PRE    1: those two calls at n = 8 in the n = 8 one pass
 *                    (default: as two calls, measured faster)
 * Every route computes the same results up to fp32 summation order (the
 * fused calls' X_next and F_pre_next bitwise).  The workspace-size functions
 * answer for the routes selected at the time they are called, so set
 * overrides before sizing a workspace.  Not thread-safe against concurrent
 * calls.  Values above 2^31 - 1 are taken as 2^31 - 1.  mhc_tuning_set
 * returns MHC_ERR_INVALID_ARG for an unknown key. */
int mhc_tuning_set(const char *name, int64_t value);
void mhc_tuning_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H */
