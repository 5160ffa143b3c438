// C ABI of libmhc (declared in include/mhc.h): host-side argument checks,
// then the kernel launches.  Nothing here allocates, synchronises or prints.
#include "mhc.h"
#include "mhc_launch.h"

#include <stdint.h>
#include <atomic>
#include <cstring>

namespace {

// Largest problem accepted: B*n*C elements below 2^40 and K = n*C below 2^30
// keep every byte offset and every 32-bit kernel index in range.
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kMaxK = int64_t(1) << 30;
constexpr int64_t kMaxB = (int64_t(1) << 31) - 1;

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void *p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes};
}

bool overlaps(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_n(int32_t n) { return n == 1 || n == 2 || n == 4 || n == 8; }

// Shape checks common to every call.  Returns MHC_OK when the shape is
// acceptable (B may be 0).
int check_shape(int64_t B, int32_t n, int64_t C) {
  if (B < 0 || n < 1 || C < 1) return MHC_ERR_INVALID_ARG;
  if (!supported_n(n) || C % 8 != 0) return MHC_ERR_UNSUPPORTED;
  // C is compared before it is multiplied: n * C itself could overflow.
  if (B > kMaxB || C > kMaxK / n || (B > 0 && B > kMaxElems / ((int64_t)n * C)))
    return MHC_ERR_UNSUPPORTED;
  return MHC_OK;
}

int64_t ncoef(int32_t n) { return (int64_t)n * n + 2 * (int64_t)n; }

int from_hip(hipError_t e) { return e == hipSuccess ? MHC_OK : MHC_ERR_HIP; }

// The element types of a call: the residual stream in bf16 (2 bytes) or E4M3
// (1 byte, the *_fp8 entry points, which need C % 16 == 0 for 16-byte
// vectors); phi in bf16 or fp32 (the *_phi32 entry points, bf16 stream).
struct Elt {
  bool fp8;
  bool phi32;
  // The workspace is the array of mhc_post_res_coeffs_pre_noalloc: routes
  // whose workspace would not fit it give way to ones that do.
  bool capped = false;
  size_t bytes() const { return fp8 ? 1 : 2; }
  size_t phi_bytes() const { return phi32 ? 4 : 2; }
};

int check_shape_elt(int64_t B, int32_t n, int64_t C, Elt e) {
  const int st = check_shape(B, n, C);
  if (st != MHC_OK) return st;
  if (e.fp8 && C % 16 != 0) return MHC_ERR_UNSUPPORTED;
  return MHC_OK;
}

// Which kernels mhc_coeffs(_fp8) runs: the one-launch small-B kernel, the
// split-K product (X staged through LDS, bf16 or E4M3; or with
// MHC_GEMM_ALGO=0 its register path) + combine, or the persistent product
// kernel of mhc_post_res_fused.hip (product-only mode, fixed-slice layout) +
// combine.  Above the small-B sizes, bf16 X at n <= 4 takes the persistent
// kernel: measured on MI355X in the three-call sequence (after mhc_post_res,
// before mhc_pre) at n=4, C=7168, B=16384 it takes 174.5 us per call against
// 201-204 for the split-K product (its 16 waves per CU keep more loads in
// flight than the split-K kernel's 4).  E4M3 X keeps the split-K product
// (116-126 against 118-137 us) and n = 8 too (the persistent kernel cannot
// hold 80-column phi operands in registers).  The persistent kernel walks
// each stream in 32-channel k-steps, so it needs C % 32 == 0; with
// MHC_GEMM_ALGO=2 other hidden sizes take the small-B kernel at any B (it is
// correct for every shape, only slower at large B).
// The product-only mode of the n = 8 pass (mhc_onepass8.hip: phi held in
// registers per 128-channel slice) runs with MHC_GEMM_ALGO=3 (bf16, n = 8,
// C <= 4096); at n=8, C=4096, B=8192 it measured 145-153 us against 141 for
// the split-K product, which stays the default.
enum class CoeffsPath { kSmall, kSplitK, kPersistent, kPass8 };

CoeffsPath coeffs_path(int64_t B, int32_t n, int64_t C, Elt e) {
  if (mhc::use_coeffs_small(B, n, C)) return CoeffsPath::kSmall;
  if (e.phi32) return CoeffsPath::kSplitK;  // fp32 phi: small-B kernel or split-K through LDS
  const int64_t algo = mhc::tune(mhc::kTuneGemmAlgo);
  if (algo == 2) return C % 32 == 0 ? CoeffsPath::kPersistent : CoeffsPath::kSmall;
  if (algo == 0 || algo == 1) return CoeffsPath::kSplitK;
  if (algo == 3) return n == 8 && !e.fp8 && mhc::onepass8_fits(B, C) ? CoeffsPath::kPass8 : CoeffsPath::kSplitK;
  if (!e.fp8 && n <= 4 && C % 32 == 0 && mhc::fixed_layout_fits(n, C)) return CoeffsPath::kPersistent;
  return CoeffsPath::kSplitK;
}

// Grid of the n = 8 pass without the hand-off: whole row tiles per round
// (each workgroup keeps one slice), as many as can be resident; no workgroup
// waits for another, so a grid larger than what is resident is only slower.
int64_t pass8_grid(const mhc::FusedPlan &p, bool apply, hipStream_t s) {
  const int64_t units = p.row_tiles * p.split;
  int64_t g = mhc::pre_mode_grid(units, p.split, mhc::onepass8_resident(apply, false, s), mhc::tune(mhc::kTuneFusedWgs));
  if (g == 0) g = p.split <= units ? p.split : units;
  return g;
}

mhc::GemmPlan split_plan(int64_t B, int32_t n, int64_t C, Elt e) {
  return mhc::plan_gemm(B, n, C, e.fp8, e.phi32);
}

size_t coeffs_ws_bytes(int64_t B, int32_t n, int64_t C, Elt e) {
  switch (coeffs_path(B, n, C, e)) {
    case CoeffsPath::kSmall: return mhc::plan_coeffs_small(B, n, C).total_bytes;
    case CoeffsPath::kPersistent: return mhc::plan_post_res_next(B, n, C, false, true).total_bytes;
    case CoeffsPath::kPass8: return mhc::plan_onepass8(B, C, false).total_bytes;
    default: return mhc::gemm_workspace_bytes(split_plan(B, n, C, e), B, n);
  }
}

int coeffs_impl(Elt e, int64_t B, int32_t n, int64_t C, const void *X_t, const void *phi,
                float alpha_pre, float alpha_post, float alpha_res, const float *b_pre,
                const float *b_post, const float *b_res, float *logits, float *r, float *H,
                void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_shape_elt(B, n, C, e);
  if (st != MHC_OK) return st;
  if (B == 0) return MHC_OK;
  if (!X_t || !phi || !b_pre || !b_post || !b_res || !logits || !r || !H || !workspace)
    return MHC_ERR_INVALID_ARG;
  if (!aligned(X_t, 16) || !aligned(phi, 16) || !aligned(workspace, 16) || !aligned(b_pre, 4) ||
      !aligned(b_post, 4) || !aligned(b_res, 4) || !aligned(logits, 4) || !aligned(r, 4) ||
      !aligned(H, 4))
    return MHC_ERR_UNSUPPORTED;

  const CoeffsPath path = coeffs_path(B, n, C, e);
  const size_t ws_need = coeffs_ws_bytes(B, n, C, e);
  const int64_t N = ncoef(n), K = (int64_t)n * C;
  const Span in[] = {span(X_t, (size_t)B * K * e.bytes()), span(phi, (size_t)K * N * e.phi_bytes()),
                     span(b_pre, (size_t)n * 4), span(b_post, (size_t)n * 4),
                     span(b_res, (size_t)n * n * 4)};
  const Span out[] = {span(logits, (size_t)B * N * 4), span(r, (size_t)B * 4),
                      span(H, (size_t)B * N * 4), span(workspace, ws_need)};
  for (const Span &o : out) {
    for (const Span &i : in)
      if (overlaps(o, i)) return MHC_ERR_INVALID_ARG;
  }
  for (int a = 0; a < 4; ++a)
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(out[a], out[b])) return MHC_ERR_INVALID_ARG;
  if (workspace_bytes < ws_need) return MHC_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (path == CoeffsPath::kSmall)
    return from_hip(mhc::launch_coeffs_small(mhc::plan_coeffs_small(B, n, C), n, e.fp8, B, C, X_t,
                                             phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post,
                                             b_res, logits, r, H, workspace, s, e.phi32));
  if (path == CoeffsPath::kPass8) {
    const mhc::FusedPlan plan = mhc::plan_onepass8(B, C, false);
    st = from_hip(mhc::launch_onepass8(plan, false, B, C, X_t, nullptr, nullptr, nullptr, phi, workspace,
                                       pass8_grid(plan, false, s), s, nullptr));
    if (st != MHC_OK) return st;
    return from_hip(mhc::launch_coeff_sinkhorn(n, B, C, plan.split, static_cast<const float *>(workspace),
                                               alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                                               logits, r, H, s, /*tree=*/true));
  }
  if (path == CoeffsPath::kPersistent) {
    const mhc::FusedPlan plan = mhc::plan_post_res_next(B, n, C, false, true);
    st = from_hip(mhc::launch_post_res_next(plan, n, e.fp8 ? mhc::kFusedCoeffsFp8 : mhc::kFusedCoeffsBf16,
                                            B, C, X_t, nullptr, nullptr, nullptr, phi, workspace, s));
    if (st != MHC_OK) return st;
    return from_hip(mhc::launch_coeff_sinkhorn(n, B, C, plan.split, static_cast<const float *>(workspace),
                                               alpha_pre, alpha_post, alpha_res, b_pre, b_post,
                                               b_res, logits, r, H, s));
  }
  const mhc::GemmPlan plan = split_plan(B, n, C, e);
  float *ws = static_cast<float *>(workspace);
  st = from_hip(mhc::launch_gemm_rms(plan, n, B, C, X_t, phi, ws, s));
  if (st != MHC_OK) return st;
  return from_hip(mhc::launch_coeff_sinkhorn(n, B, C, plan.split, ws, alpha_pre, alpha_post,
                                             alpha_res, b_pre, b_post, b_res, logits, r, H, s));
}

int pre_impl(Elt e, int64_t B, int32_t n, int64_t C, const void *X_t, const float *H,
             void *F_pre, void *stream) {
  int st = check_shape_elt(B, n, C, e);
  if (st != MHC_OK) return st;
  if (B == 0) return MHC_OK;
  if (!X_t || !H || !F_pre) return MHC_ERR_INVALID_ARG;
  if (!aligned(X_t, 16) || !aligned(F_pre, 16) || !aligned(H, 4)) return MHC_ERR_UNSUPPORTED;
  const int64_t N = ncoef(n);
  const Span o = span(F_pre, (size_t)B * C * e.bytes());
  if (overlaps(o, span(X_t, (size_t)B * n * C * e.bytes())) || overlaps(o, span(H, (size_t)B * N * 4)))
    return MHC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(e.fp8 ? mhc::launch_pre_fp8(n, B, C, X_t, H, F_pre, s)
                        : mhc::launch_pre(n, B, C, X_t, H, F_pre, s));
}

int post_res_impl(Elt e, int64_t B, int32_t n, int64_t C, const void *X_t, const void *F_out,
                  const float *H, void *X_next, void *stream) {
  int st = check_shape_elt(B, n, C, e);
  if (st != MHC_OK) return st;
  if (B == 0) return MHC_OK;
  if (!X_t || !F_out || !H || !X_next) return MHC_ERR_INVALID_ARG;
  if (!aligned(X_t, 16) || !aligned(F_out, 16) || !aligned(X_next, 16) || !aligned(H, 4))
    return MHC_ERR_UNSUPPORTED;
  const int64_t N = ncoef(n);
  const Span o = span(X_next, (size_t)B * n * C * e.bytes());
  if (overlaps(o, span(X_t, (size_t)B * n * C * e.bytes())) ||
      overlaps(o, span(F_out, (size_t)B * C * e.bytes())) || overlaps(o, span(H, (size_t)B * N * 4)))
    return MHC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(e.fp8 ? mhc::launch_post_res_fp8(n, B, C, X_t, F_out, H, X_next, s)
                        : mhc::launch_post_res(n, B, C, X_t, F_out, H, X_next, s));
}

// How mhc_post_res_coeffs(_fp8) runs: small B -> the apply, then the
// one-launch small-B coefficient kernel on X_next; otherwise the fused kernel,
// except where the apply followed by the split-K product on X_next measured
// faster (MI355X):
//   n = 8: the fused kernel re-reads 80-column phi blocks from L2 for every 16
//          rows (501 vs 321 us bf16 at B=8192, C=4096); MHC_FUSED_N8=1 forces it;
//   E4M3:  outside the fixed-slice layout (phi operands held in registers)
//          the fused kernel's per-step phi reads from L2 cost more than the
//          second pass saves; in it the fused kernel wins (243 vs 288 us per
//          call, 371 vs 383 us per layer with pre_fp8, chained layers at
//          n=4, C=7168, B=16384).  MHC_FUSED_FP8=1 forces the fused kernel,
//          MHC_FUSED_FP8=0 the two passes.
//   n = 8, bf16: the n = 8 pass (mhc_onepass8.hip) where it fits (C <= 4096);
//          MHC_FUSED_N8=0 forces the two passes.
enum class FusedRoute { kSmall, kTwoPass, kFused, kPass8 };

FusedRoute fused_route(int64_t B, int32_t n, int64_t C, Elt e) {
  if (mhc::use_coeffs_small(B, n, C)) return FusedRoute::kSmall;
  if (e.phi32) return FusedRoute::kTwoPass;  // the fused kernel takes bf16 phi only
  if (n == 8) {
    const int64_t v = mhc::tune(mhc::kTuneFusedN8);
    if (v < 0 && !e.fp8 && mhc::onepass8_fits(B, C) &&
        !(e.capped && mhc::plan_onepass8(B, C, false).total_bytes > (size_t)MHC_NOALLOC_SCRATCH_BYTES))
      return FusedRoute::kPass8;
    if (v <= 0) return FusedRoute::kTwoPass;
  }
  if (e.fp8) {
    const int64_t v = mhc::tune(mhc::kTuneFusedFp8);
    if (v >= 0) return v == 0 ? FusedRoute::kTwoPass : FusedRoute::kFused;
    if (!mhc::plan_post_res_next(B, n, C, false, true).fixed) return FusedRoute::kTwoPass;
  }
  return FusedRoute::kFused;
}

size_t post_res_coeffs_ws_bytes(int64_t B, int32_t n, int64_t C, Elt e) {
  if (check_shape_elt(B, n, C, e) != MHC_OK || B == 0 || C % 32 != 0) return 0;
  switch (fused_route(B, n, C, e)) {
    case FusedRoute::kSmall: return mhc::plan_coeffs_small(B, n, C).total_bytes;
    case FusedRoute::kTwoPass: return mhc::gemm_workspace_bytes(split_plan(B, n, C, e), B, n);
    case FusedRoute::kPass8: return mhc::plan_onepass8(B, C, false).total_bytes;
    default: return mhc::plan_post_res_next(B, n, C, false, e.fp8).total_bytes;
  }
}

// mhc_post_res_coeffs_pre(_fp8): the fused kernel's pre-mix mode (one pass
// that also writes the next layer's F_pre) wherever mhc_post_res_coeffs(_fp8)
// would run the fused kernel and the mode fits the shape (n <= 4, at most 16
// 512-channel steps per row); otherwise mhc_post_res_coeffs(_fp8) followed by
// mhc_pre(_fp8) on X_next.  MHC_FUSED_PRE=0 forces the latter.
bool pre_fused(int64_t B, int32_t n, int64_t C, Elt e) {
  if (e.phi32) return false;
  if (mhc::tune(mhc::kTuneFusedPre) == 0) return false;
  const FusedRoute route = fused_route(B, n, C, e);
  // n = 8: the pass with the hand-off (one register set of loads beside it)
  // measured slower than its two calls at n=8, C=4096, B=8192 (461-546
  // against 360-392 us per layer), so it runs only with MHC_PASS8_PRE=1.
  if (route == FusedRoute::kPass8) return mhc::tune(mhc::kTunePass8Pre) > 0;
  return route == FusedRoute::kFused && mhc::pre_mode_fits(B, n, C);
}

// Workspace layout of a one-pass shape (records and give-up word included).
mhc::FusedPlan pre_plan(int64_t B, int32_t n, int64_t C, Elt e) {
  return n == 8 ? mhc::plan_onepass8(B, C, true) : mhc::plan_post_res_next(B, n, C, true, e.fp8);
}

// The single-slice route (mhc_layer_small.hip): bf16, n <= 4, the small-B
// sizes, n*C <= 1024, wherever the one-pass calls are not turned off.  It
// needs no workspace (the two calls' size is still asked for) and never waits.
bool small_pass(int64_t B, int32_t n, int64_t C, Elt e) {
  if (e.fp8 || e.phi32) return false;
  if (mhc::tune(mhc::kTuneFusedPre) == 0) return false;
  return mhc::layer_small_fits(B, n, C);
}

size_t post_res_coeffs_pre_ws_bytes(int64_t B, int32_t n, int64_t C, Elt e) {
  if (check_shape_elt(B, n, C, e) != MHC_OK || B == 0 || C % 32 != 0) return 0;
  if (pre_fused(B, n, C, e)) return pre_plan(B, n, C, e).total_bytes;
  return post_res_coeffs_ws_bytes(B, n, C, e);
}

// F_pre_next: null for mhc_post_res_coeffs(_fp8, _phi32); the output of
// mhc_post_res_coeffs_pre(_fp8) otherwise.
int post_res_coeffs_impl(Elt e, int64_t B, int32_t n, int64_t C, const void *X_t,
                         const void *F_out, const float *H, void *X_next, const void *phi_next,
                         float alpha_pre, float alpha_post, float alpha_res, const float *b_pre,
                         const float *b_post, const float *b_res, float *logits_next,
                         float *r_next, float *H_next, void *workspace, size_t workspace_bytes,
                         void *stream, bool with_pre = false, void *F_pre_next = nullptr) {
  int st = check_shape_elt(B, n, C, e);
  if (st != MHC_OK) return st;
  if (C % 32 != 0) return MHC_ERR_UNSUPPORTED;
  if (B == 0) return MHC_OK;
  if (!X_t || !F_out || !H || !X_next || !phi_next || !b_pre || !b_post || !b_res ||
      !logits_next || !r_next || !H_next || !workspace || (with_pre && !F_pre_next))
    return MHC_ERR_INVALID_ARG;
  if (!aligned(X_t, 16) || !aligned(F_out, 16) || !aligned(X_next, 16) || !aligned(phi_next, 16) ||
      !aligned(workspace, 16) || !aligned(H, 4) || !aligned(b_pre, 4) || !aligned(b_post, 4) ||
      !aligned(b_res, 4) || !aligned(logits_next, 4) || !aligned(r_next, 4) || !aligned(H_next, 4) ||
      (with_pre && !aligned(F_pre_next, 16)))
    return MHC_ERR_UNSUPPORTED;
  const FusedRoute route = fused_route(B, n, C, e);
  bool one_pass = with_pre && pre_fused(B, n, C, e);
  const mhc::FusedPlan plan = route == FusedRoute::kPass8 ? mhc::plan_onepass8(B, C, one_pass)
                                                           : mhc::plan_post_res_next(B, n, C, one_pass, e.fp8);
  const size_t ws_need = with_pre ? post_res_coeffs_pre_ws_bytes(B, n, C, e) : post_res_coeffs_ws_bytes(B, n, C, e);
  const int64_t N = ncoef(n), K = (int64_t)n * C;
  const size_t eb = e.bytes();
  const Span in[] = {span(X_t, (size_t)B * K * eb), span(F_out, (size_t)B * C * eb),
                     span(H, (size_t)B * N * 4), span(phi_next, (size_t)K * N * e.phi_bytes()),
                     span(b_pre, (size_t)n * 4), span(b_post, (size_t)n * 4),
                     span(b_res, (size_t)n * n * 4)};
  const Span out[] = {span(X_next, (size_t)B * K * eb), span(logits_next, (size_t)B * N * 4),
                      span(r_next, (size_t)B * 4), span(H_next, (size_t)B * N * 4),
                      span(workspace, ws_need),
                      with_pre ? span(F_pre_next, (size_t)B * C * eb) : Span{0, 0}};
  for (const Span &o : out)
    for (const Span &i : in)
      if (overlaps(o, i)) return MHC_ERR_INVALID_ARG;
  for (int a = 0; a < 6; ++a)
    for (int b = a + 1; b < 6; ++b)
      if (overlaps(out[a], out[b])) return MHC_ERR_INVALID_ARG;
  if (workspace_bytes < ws_need) return MHC_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (with_pre && small_pass(B, n, C, e))  // one kernel: apply, coefficients and F_pre
    return from_hip(mhc::launch_layer_small(n, true, B, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                                            alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                                            F_pre_next, s));
  int64_t grid = 0;
  if (one_pass) {
    // The pass needs every workgroup of a round resident at once: size the
    // grid from what the device and the stream's CUs hold, and run the two
    // calls instead when not even one row tile's slices fit together.
    grid = mhc::pre_mode_grid(plan.row_tiles * plan.split, plan.split,
                              route == FusedRoute::kPass8
                                  ? mhc::onepass8_resident(true, true, s)
                                  : mhc::pre_mode_resident(n, e.fp8 ? mhc::kFusedApplyPreFp8 : mhc::kFusedApplyPreBf16, s),
                              mhc::tune(mhc::kTuneFusedWgs));
    if (grid == 0) {
      one_pass = false;
      // The give-up word then reports no give-up.
      st = from_hip(mhc::launch_zero(static_cast<char *>(workspace) + plan.flag_offset, 16, s));
      if (st != MHC_OK) return st;
    }
  }
  if (one_pass) {
    const mhc::PreOut po{F_pre_next, b_pre, alpha_pre, grid};
    if (route == FusedRoute::kPass8)
      st = from_hip(mhc::launch_onepass8(plan, true, B, C, X_t, F_out, H, X_next, phi_next, workspace, grid, s, &po));
    else
      st = from_hip(mhc::launch_post_res_next(plan, n, e.fp8 ? mhc::kFusedApplyPreFp8 : mhc::kFusedApplyPreBf16,
                                              B, C, X_t, F_out, H, X_next, phi_next, workspace, s, &po));
    if (st != MHC_OK) return st;
    return from_hip(mhc::launch_coeff_sinkhorn(n, B, C, plan.split, static_cast<const float *>(workspace),
                                               alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                                               logits_next, r_next, H_next, s, /*tree=*/true));
  }
  if (with_pre) {
    // Not one pass: the coefficient call, then the pre-mix of X_next.
    st = post_res_coeffs_impl(e, B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre, alpha_post,
                              alpha_res, b_pre, b_post, b_res, logits_next, r_next, H_next,
                              workspace, workspace_bytes, stream);
    if (st != MHC_OK) return st;
    return from_hip(e.fp8 ? mhc::launch_pre_fp8(n, B, C, X_next, H_next, F_pre_next, s)
                          : mhc::launch_pre(n, B, C, X_next, H_next, F_pre_next, s));
  }
  if (route == FusedRoute::kPass8) {
    st = from_hip(mhc::launch_onepass8(plan, true, B, C, X_t, F_out, H, X_next, phi_next, workspace,
                                       pass8_grid(plan, true, s), s, nullptr));
    if (st != MHC_OK) return st;
    return from_hip(mhc::launch_coeff_sinkhorn(n, B, C, plan.split, static_cast<const float *>(workspace),
                                               alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                                               logits_next, r_next, H_next, s, /*tree=*/true));
  }
  if (route != FusedRoute::kFused) {
    if (route == FusedRoute::kSmall && !e.fp8 && !e.phi32 && mhc::tune(mhc::kTuneApplySmall) != 0 &&
        mhc::apply_coeffs_small_fits(B, n, C))  // the apply and the coefficients in one kernel
      return from_hip(mhc::launch_apply_coeffs_small(mhc::plan_coeffs_small(B, n, C), n, B, C, X_t, F_out, H,
                                                     X_next, phi_next, alpha_pre, alpha_post, alpha_res, b_pre,
                                                     b_post, b_res, logits_next, r_next, H_next, workspace, s));
    st = from_hip(e.fp8 ? mhc::launch_post_res_fp8(n, B, C, X_t, F_out, H, X_next, s)
                        : mhc::launch_post_res(n, B, C, X_t, F_out, H, X_next, s));
    if (st != MHC_OK) return st;
    if (route == FusedRoute::kSmall)
      return from_hip(mhc::launch_coeffs_small(mhc::plan_coeffs_small(B, n, C), n, e.fp8, B, C,
                                               X_next, phi_next, alpha_pre, alpha_post, alpha_res,
                                               b_pre, b_post, b_res, logits_next, r_next, H_next,
                                               workspace, s, e.phi32));
    const mhc::GemmPlan gp = split_plan(B, n, C, e);
    float *ws = static_cast<float *>(workspace);
    st = from_hip(mhc::launch_gemm_rms(gp, n, B, C, X_next, phi_next, ws, s));
    if (st != MHC_OK) return st;
    return from_hip(mhc::launch_coeff_sinkhorn(n, B, C, gp.split, ws, alpha_pre, alpha_post,
                                               alpha_res, b_pre, b_post, b_res, logits_next,
                                               r_next, H_next, s));
  }
  st = from_hip(mhc::launch_post_res_next(plan, n, e.fp8 ? mhc::kFusedApplyFp8 : mhc::kFusedApplyBf16,
                                          B, C, X_t, F_out, H, X_next, phi_next, workspace, s));
  if (st != MHC_OK) return st;
  return from_hip(mhc::launch_coeff_sinkhorn(n, B, C, plan.split, static_cast<const float *>(workspace),
                                             alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                                             logits_next, r_next, H_next, s));
}

// mhc_coeffs_pre(_fp8): the product-only pre-mix mode of the fused kernel
// (X_t read once for the logits, the sums of squares and F_pre) wherever
// mhc_post_res_coeffs_pre(_fp8) takes its one pass; otherwise mhc_coeffs(_fp8)
// followed by mhc_pre(_fp8).  The workspace of a one-pass shape holds the
// pre-mix layout (give-up word included) and also mhc_coeffs's workspace,
// for the two calls that run when the grid cannot be resident.
bool coeffs_pre_fused(int64_t B, int32_t n, int64_t C, Elt e) { return C % 32 == 0 && pre_fused(B, n, C, e); }

size_t coeffs_pre_ws_bytes(int64_t B, int32_t n, int64_t C, Elt e) {
  if (check_shape_elt(B, n, C, e) != MHC_OK || B == 0) return 0;
  const size_t two = coeffs_ws_bytes(B, n, C, e);
  if (!coeffs_pre_fused(B, n, C, e)) return two;
  const size_t one = pre_plan(B, n, C, e).total_bytes;
  return one > two ? one : two;
}

int coeffs_pre_impl(Elt e, int64_t B, int32_t n, int64_t C, const void *X_t, const void *phi,
                    float alpha_pre, float alpha_post, float alpha_res, const float *b_pre,
                    const float *b_post, const float *b_res, float *logits, float *r, float *H,
                    void *F_pre, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_shape_elt(B, n, C, e);
  if (st != MHC_OK) return st;
  if (B == 0) return MHC_OK;
  if (!X_t || !phi || !b_pre || !b_post || !b_res || !logits || !r || !H || !F_pre || !workspace)
    return MHC_ERR_INVALID_ARG;
  if (!aligned(X_t, 16) || !aligned(phi, 16) || !aligned(workspace, 16) || !aligned(F_pre, 16) ||
      !aligned(b_pre, 4) || !aligned(b_post, 4) || !aligned(b_res, 4) || !aligned(logits, 4) ||
      !aligned(r, 4) || !aligned(H, 4))
    return MHC_ERR_UNSUPPORTED;
  bool one_pass = coeffs_pre_fused(B, n, C, e);
  const size_t ws_need = coeffs_pre_ws_bytes(B, n, C, e);
  const int64_t N = ncoef(n), K = (int64_t)n * C;
  const Span in[] = {span(X_t, (size_t)B * K * e.bytes()), span(phi, (size_t)K * N * e.phi_bytes()),
                     span(b_pre, (size_t)n * 4), span(b_post, (size_t)n * 4),
                     span(b_res, (size_t)n * n * 4)};
  const Span out[] = {span(logits, (size_t)B * N * 4), span(r, (size_t)B * 4),
                      span(H, (size_t)B * N * 4), span(workspace, ws_need),
                      span(F_pre, (size_t)B * C * e.bytes())};
  for (const Span &o : out)
    for (const Span &i : in)
      if (overlaps(o, i)) return MHC_ERR_INVALID_ARG;
  for (int a = 0; a < 5; ++a)
    for (int b = a + 1; b < 5; ++b)
      if (overlaps(out[a], out[b])) return MHC_ERR_INVALID_ARG;
  if (workspace_bytes < ws_need) return MHC_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mode = e.fp8 ? mhc::kFusedCoeffsPreFp8 : mhc::kFusedCoeffsPreBf16;
  if (small_pass(B, n, C, e))  // one kernel: coefficients and F_pre
    return from_hip(mhc::launch_layer_small(n, false, B, C, X_t, nullptr, nullptr, nullptr, phi, alpha_pre,
                                            alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, F_pre, s));
  if (one_pass) {
    // As in mhc_post_res_coeffs_pre: a grid that can be resident at once,
    // else the two calls (the give-up word then reports no give-up).
    const mhc::FusedPlan plan = pre_plan(B, n, C, e);
    const int64_t grid = mhc::pre_mode_grid(plan.row_tiles * plan.split, plan.split,
                                            n == 8 ? mhc::onepass8_resident(false, true, s)
                                                   : mhc::pre_mode_resident(n, mode, s),
                                            mhc::tune(mhc::kTuneFusedWgs));
    if (grid > 0) {
      const mhc::PreOut po{F_pre, b_pre, alpha_pre, grid};
      if (n == 8)
        st = from_hip(mhc::launch_onepass8(plan, false, B, C, X_t, nullptr, nullptr, nullptr, phi, workspace,
                                           grid, s, &po));
      else
        st = from_hip(mhc::launch_post_res_next(plan, n, mode, B, C, X_t, nullptr, nullptr, nullptr, phi,
                                                workspace, s, &po));
      if (st != MHC_OK) return st;
      return from_hip(mhc::launch_coeff_sinkhorn(n, B, C, plan.split, static_cast<const float *>(workspace),
                                                 alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                                                 logits, r, H, s, /*tree=*/true));
    }
    one_pass = false;
    st = from_hip(mhc::launch_zero(static_cast<char *>(workspace) + plan.flag_offset, 16, s));
    if (st != MHC_OK) return st;
  }
  st = coeffs_impl(e, B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res,
                   logits, r, H, workspace, workspace_bytes, stream);
  if (st != MHC_OK) return st;
  return from_hip(e.fp8 ? mhc::launch_pre_fp8(n, B, C, X_t, H, F_pre, s)
                        : mhc::launch_pre(n, B, C, X_t, H, F_pre, s));
}

// The give-up word of a one-pass workspace (pre-mix layout): MHC_OK while
// zero, MHC_ERR_INCOMPLETE once a wait gave up.  Synchronises the stream.
int read_giveup(int64_t B, int32_t n, int64_t C, Elt e, const void *workspace, void *stream) {
  const mhc::FusedPlan plan = pre_plan(B, n, C, e);
  uint32_t word = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(&word, static_cast<const char *>(workspace) + plan.flag_offset, sizeof(word),
                     hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MHC_ERR_HIP;
  return word == 0 ? MHC_OK : MHC_ERR_INCOMPLETE;
}

constexpr Elt kBf16{false, false}, kFp8{true, false}, kPhi32{false, true};
constexpr Elt kBf16Capped{false, false, true};  // bf16 in the no-alloc array

// Route and launch-shape overrides (mhc_tuning_set): -1 = unset.
std::atomic<int64_t> g_tune[mhc::kTuneCount] = {};
std::atomic<bool> g_tune_init{false};

struct TuneName {
  const char *name;
  mhc::TuneKey key;
};
constexpr TuneName kTuneNames[] = {
    {"MHC_SMALL_MAX_B", mhc::kTuneSmallMaxB}, {"MHC_GEMM_ALGO", mhc::kTuneGemmAlgo},
    {"MHC_SPLIT_K", mhc::kTuneSplitK},        {"MHC_GEMM_WGS", mhc::kTuneGemmWgs},
    {"MHC_GEMM_MB", mhc::kTuneGemmMb},        {"MHC_FUSED_N8", mhc::kTuneFusedN8},
    {"MHC_FUSED_FP8", mhc::kTuneFusedFp8},    {"MHC_FUSED_FIXED", mhc::kTuneFusedFixed},
    {"MHC_FUSED_SPU", mhc::kTuneFusedSpu},    {"MHC_FUSED_WGS", mhc::kTuneFusedWgs},
    {"MHC_FUSED_PRE", mhc::kTuneFusedPre},    {"MHC_LPN_ALGO", mhc::kTuneLpnAlgo},
    {"MHC_GEMM_KC", mhc::kTuneGemmKc},        {"MHC_GEMM_STAGES", mhc::kTuneGemmStages},
    {"MHC_GEMM_WAVES", mhc::kTuneGemmWaves},  {"MHC_GEMM_XREG", mhc::kTuneGemmXreg},
    {"MHC_APPLY_SMALL", mhc::kTuneApplySmall},
    {"MHC_PASS8_SETS", mhc::kTunePass8Sets},  {"MHC_PASS8_PRE", mhc::kTunePass8Pre},
};
static_assert(sizeof(kTuneNames) / sizeof(kTuneNames[0]) == mhc::kTuneCount, "one name per key");

void tune_reset_all() {
  for (auto &v : g_tune) v.store(-1, std::memory_order_relaxed);
}

void tune_init() {
  if (!g_tune_init.load(std::memory_order_acquire)) {
    tune_reset_all();
    g_tune_init.store(true, std::memory_order_release);
  }
}

// Workspace of mhc_post_res_coeffs_pre_noalloc: a device array of fixed size,
// one copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address (in host code it names a host-side stand-in);
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current.
constexpr size_t kNoAllocScratchBytes = MHC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MHC_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MHC_ERR_UNSUPPORTED;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // Any thread that gets here resolves the same address; the first store wins.
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MHC_ERR_HIP;
    void *expected = nullptr;
    g_scratch_ptr[dev].compare_exchange_strong(expected, p, std::memory_order_acq_rel);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  }
  *out = p;
  return MHC_OK;
}

}  // namespace

namespace mhc {
int64_t tune(TuneKey k) {
  if (!g_tune_init.load(std::memory_order_acquire)) return -1;
  return g_tune[k].load(std::memory_order_relaxed);
}
}  // namespace mhc

extern "C" {

const char *mhc_status_string(int status) {
  switch (status) {
    case MHC_OK: return "MHC_OK";
    case MHC_ERR_INVALID_ARG: return "MHC_ERR_INVALID_ARG: null pointer, negative size or overlapping buffers";
    case MHC_ERR_UNSUPPORTED: return "MHC_ERR_UNSUPPORTED: n not in {1,2,4,8}, C % 8 != 0 (C % 16 for E4M3, C % 32 for the fused call), size too large or misaligned pointer";
    case MHC_ERR_WORKSPACE: return "MHC_ERR_WORKSPACE: workspace smaller than the call's workspace-size function returns";
    case MHC_ERR_HIP: return "MHC_ERR_HIP: the HIP runtime reported an error";
    case MHC_ERR_INCOMPLETE: return "MHC_ERR_INCOMPLETE: a one-pass call gave up waiting for another workgroup; its F_pre_next holds NaN where it gave up";
    default: return "MHC_ERR_UNKNOWN";
  }
}

int mhc_tuning_set(const char *name, int64_t value) {
  if (!name) return MHC_ERR_INVALID_ARG;
  tune_init();
  for (const TuneName &t : kTuneNames)
    if (std::strcmp(t.name, name) == 0) {
      // Values are clamped to 2^31 - 1, far above any meaningful setting,
      // so the launch-shape arithmetic they enter cannot overflow.
      constexpr int64_t kMaxTune = (int64_t(1) << 31) - 1;
      g_tune[t.key].store(value < 0 ? -1 : (value > kMaxTune ? kMaxTune : value), std::memory_order_relaxed);
      return MHC_OK;
    }
  return MHC_ERR_INVALID_ARG;
}

void mhc_tuning_reset(void) {
  tune_init();
  tune_reset_all();
}

size_t mhc_coeffs_workspace_size(int64_t B, int32_t n, int64_t C) {
  if (check_shape(B, n, C) != MHC_OK || B == 0) return 0;
  return coeffs_ws_bytes(B, n, C, kBf16);
}

int32_t mhc_coeffs_split_k(int64_t B, int32_t n, int64_t C) {
  if (check_shape(B, n, C) != MHC_OK || B == 0) return 0;
  switch (coeffs_path(B, n, C, kBf16)) {
    case CoeffsPath::kSmall: return mhc::plan_coeffs_small(B, n, C).split;
    case CoeffsPath::kPersistent: return mhc::plan_post_res_next(B, n, C, false, true).split;
    case CoeffsPath::kPass8: return mhc::plan_onepass8(B, C, false).split;
    default: return mhc::plan_gemm(B, n, C).split;
  }
}

int mhc_coeffs(int64_t B, int32_t n, int64_t C, const void *X_t, const void *phi,
               float alpha_pre, float alpha_post, float alpha_res, const float *b_pre,
               const float *b_post, const float *b_res, float *logits, float *r, float *H,
               void *workspace, size_t workspace_bytes, void *stream) {
  return coeffs_impl(kBf16, B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post,
                     b_res, logits, r, H, workspace, workspace_bytes, stream);
}

int mhc_pre(int64_t B, int32_t n, int64_t C, const void *X_t, const float *H, void *F_pre,
            void *stream) {
  return pre_impl(kBf16, B, n, C, X_t, H, F_pre, stream);
}

int mhc_post_res(int64_t B, int32_t n, int64_t C, const void *X_t, const void *F_out,
                 const float *H, void *X_next, void *stream) {
  return post_res_impl(kBf16, B, n, C, X_t, F_out, H, X_next, stream);
}

size_t mhc_coeffs_pre_workspace_size(int64_t B, int32_t n, int64_t C) {
  return coeffs_pre_ws_bytes(B, n, C, kBf16);
}

int mhc_coeffs_pre(int64_t B, int32_t n, int64_t C, const void *X_t, const void *phi,
                   float alpha_pre, float alpha_post, float alpha_res, const float *b_pre,
                   const float *b_post, const float *b_res, float *logits, float *r, float *H,
                   void *F_pre, void *workspace, size_t workspace_bytes, void *stream) {
  return coeffs_pre_impl(kBf16, B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post,
                         b_res, logits, r, H, F_pre, workspace, workspace_bytes, stream);
}

int32_t mhc_coeffs_pre_one_pass(int64_t B, int32_t n, int64_t C) {
  if (check_shape(B, n, C) != MHC_OK || B == 0) return 0;
  return coeffs_pre_fused(B, n, C, kBf16) || small_pass(B, n, C, kBf16) ? 1 : 0;
}

size_t mhc_post_res_coeffs_workspace_size(int64_t B, int32_t n, int64_t C) {
  return post_res_coeffs_ws_bytes(B, n, C, kBf16);
}

int mhc_post_res_coeffs(int64_t B, int32_t n, int64_t C, const void *X_t, const void *F_out,
                        const float *H, void *X_next, const void *phi_next, float alpha_pre,
                        float alpha_post, float alpha_res, const float *b_pre, const float *b_post,
                        const float *b_res, float *logits_next, float *r_next, float *H_next,
                        void *workspace, size_t workspace_bytes, void *stream) {
  return post_res_coeffs_impl(kBf16, B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre,
                              alpha_post, alpha_res, b_pre, b_post, b_res, logits_next, r_next,
                              H_next, workspace, workspace_bytes, stream);
}

size_t mhc_post_res_coeffs_pre_workspace_size(int64_t B, int32_t n, int64_t C) {
  return post_res_coeffs_pre_ws_bytes(B, n, C, kBf16);
}

int mhc_post_res_coeffs_pre(int64_t B, int32_t n, int64_t C, const void *X_t, const void *F_out,
                            const float *H, void *X_next, const void *phi_next, float alpha_pre,
                            float alpha_post, float alpha_res, const float *b_pre,
                            const float *b_post, const float *b_res, float *logits_next,
                            float *r_next, float *H_next, void *F_pre_next, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return post_res_coeffs_impl(kBf16, B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre,
                              alpha_post, alpha_res, b_pre, b_post, b_res, logits_next, r_next,
                              H_next, workspace, workspace_bytes, stream, true, F_pre_next);
}

int mhc_post_res_coeffs_pre_check(int64_t B, int32_t n, int64_t C, int32_t fp8,
                                  const void *workspace, size_t workspace_bytes, void *stream) {
  const Elt e = fp8 ? kFp8 : (workspace ? kBf16 : kBf16Capped);
  const int st = check_shape_elt(B, n, C, e);
  if (st != MHC_OK) return st;
  if (C % 32 != 0) return MHC_ERR_UNSUPPORTED;
  if (B == 0 || !pre_fused(B, n, C, e)) return MHC_OK;  // the two calls and the single-slice kernel never give up
  if (!workspace) {  // the array of mhc_post_res_coeffs_pre_noalloc
    if (fp8) return MHC_ERR_INVALID_ARG;
    if (post_res_coeffs_pre_ws_bytes(B, n, C, e) > kNoAllocScratchBytes) return MHC_ERR_WORKSPACE;
    void *ws = nullptr;
    const int sst = noalloc_scratch(&ws);
    if (sst != MHC_OK) return sst;
    workspace = ws;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (workspace_bytes < post_res_coeffs_pre_ws_bytes(B, n, C, e)) return MHC_ERR_WORKSPACE;
  return read_giveup(B, n, C, e, workspace, stream);
}

int mhc_coeffs_pre_check(int64_t B, int32_t n, int64_t C, int32_t fp8, const void *workspace,
                         size_t workspace_bytes, void *stream) {
  const Elt e = fp8 ? kFp8 : kBf16;
  const int st = check_shape_elt(B, n, C, e);
  if (st != MHC_OK) return st;
  if (B == 0 || !coeffs_pre_fused(B, n, C, e)) return MHC_OK;  // the two calls and the single-slice kernel never give up
  if (!workspace) return MHC_ERR_INVALID_ARG;
  if (workspace_bytes < coeffs_pre_ws_bytes(B, n, C, e)) return MHC_ERR_WORKSPACE;
  return read_giveup(B, n, C, e, workspace, stream);
}

int mhc_post_res_coeffs_pre_noalloc(int64_t B, int32_t n, int64_t C, const void *X_t,
                                    const void *F_out, const float *H, void *X_next,
                                    const void *phi_next, float alpha_pre, float alpha_post,
                                    float alpha_res, const float *b_pre, const float *b_post,
                                    const float *b_res, float *logits_next, float *r_next,
                                    float *H_next, void *F_pre_next, void *stream) {
  int st = check_shape_elt(B, n, C, kBf16);
  if (st != MHC_OK) return st;
  if (C % 32 != 0) return MHC_ERR_UNSUPPORTED;
  if (B == 0) return MHC_OK;
  if (post_res_coeffs_pre_ws_bytes(B, n, C, kBf16Capped) > kNoAllocScratchBytes) return MHC_ERR_WORKSPACE;
  void *ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != MHC_OK) return st;
  return post_res_coeffs_impl(kBf16Capped, B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre,
                              alpha_post, alpha_res, b_pre, b_post, b_res, logits_next, r_next,
                              H_next, ws, kNoAllocScratchBytes, stream, true, F_pre_next);
}

int32_t mhc_post_res_coeffs_pre_one_pass(int64_t B, int32_t n, int64_t C) {
  if (check_shape(B, n, C) != MHC_OK || B == 0 || C % 32 != 0) return 0;
  return pre_fused(B, n, C, kBf16) || small_pass(B, n, C, kBf16) ? 1 : 0;
}

size_t mhc_coeffs_fp8_workspace_size(int64_t B, int32_t n, int64_t C) {
  if (check_shape_elt(B, n, C, kFp8) != MHC_OK || B == 0) return 0;
  return coeffs_ws_bytes(B, n, C, kFp8);
}

int mhc_coeffs_fp8(int64_t B, int32_t n, int64_t C, const void *X_t, const void *phi,
                   float alpha_pre, float alpha_post, float alpha_res, const float *b_pre,
                   const float *b_post, const float *b_res, float *logits, float *r, float *H,
                   void *workspace, size_t workspace_bytes, void *stream) {
  return coeffs_impl(kFp8, B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post,
                     b_res, logits, r, H, workspace, workspace_bytes, stream);
}

int mhc_pre_fp8(int64_t B, int32_t n, int64_t C, const void *X_t, const float *H, void *F_pre,
                void *stream) {
  return pre_impl(kFp8, B, n, C, X_t, H, F_pre, stream);
}

int mhc_post_res_fp8(int64_t B, int32_t n, int64_t C, const void *X_t, const void *F_out,
                     const float *H, void *X_next, void *stream) {
  return post_res_impl(kFp8, B, n, C, X_t, F_out, H, X_next, stream);
}

size_t mhc_coeffs_pre_fp8_workspace_size(int64_t B, int32_t n, int64_t C) {
  return coeffs_pre_ws_bytes(B, n, C, kFp8);
}

int mhc_coeffs_pre_fp8(int64_t B, int32_t n, int64_t C, const void *X_t, const void *phi,
                       float alpha_pre, float alpha_post, float alpha_res, const float *b_pre,
                       const float *b_post, const float *b_res, float *logits, float *r, float *H,
                       void *F_pre, void *workspace, size_t workspace_bytes, void *stream) {
  return coeffs_pre_impl(kFp8, B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post,
                         b_res, logits, r, H, F_pre, workspace, workspace_bytes, stream);
}

int32_t mhc_coeffs_pre_fp8_one_pass(int64_t B, int32_t n, int64_t C) {
  if (check_shape_elt(B, n, C, kFp8) != MHC_OK || B == 0) return 0;
  return coeffs_pre_fused(B, n, C, kFp8) ? 1 : 0;
}

size_t mhc_post_res_coeffs_fp8_workspace_size(int64_t B, int32_t n, int64_t C) {
  return post_res_coeffs_ws_bytes(B, n, C, kFp8);
}

int mhc_post_res_coeffs_fp8(int64_t B, int32_t n, int64_t C, const void *X_t, const void *F_out,
                            const float *H, void *X_next, const void *phi_next, float alpha_pre,
                            float alpha_post, float alpha_res, const float *b_pre,
                            const float *b_post, const float *b_res, float *logits_next,
                            float *r_next, float *H_next, void *workspace, size_t workspace_bytes,
                            void *stream) {
  return post_res_coeffs_impl(kFp8, B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre,
                              alpha_post, alpha_res, b_pre, b_post, b_res, logits_next, r_next,
                              H_next, workspace, workspace_bytes, stream);
}

size_t mhc_post_res_coeffs_pre_fp8_workspace_size(int64_t B, int32_t n, int64_t C) {
  return post_res_coeffs_pre_ws_bytes(B, n, C, kFp8);
}

int mhc_post_res_coeffs_pre_fp8(int64_t B, int32_t n, int64_t C, const void *X_t,
                                const void *F_out, const float *H, void *X_next,
                                const void *phi_next, float alpha_pre, float alpha_post,
                                float alpha_res, const float *b_pre, const float *b_post,
                                const float *b_res, float *logits_next, float *r_next,
                                float *H_next, void *F_pre_next, void *workspace,
                                size_t workspace_bytes, void *stream) {
  return post_res_coeffs_impl(kFp8, B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre,
                              alpha_post, alpha_res, b_pre, b_post, b_res, logits_next, r_next,
                              H_next, workspace, workspace_bytes, stream, true, F_pre_next);
}

int32_t mhc_post_res_coeffs_pre_fp8_one_pass(int64_t B, int32_t n, int64_t C) {
  if (check_shape_elt(B, n, C, kFp8) != MHC_OK || B == 0 || C % 32 != 0) return 0;
  return pre_fused(B, n, C, kFp8) ? 1 : 0;
}

size_t mhc_coeffs_phi32_workspace_size(int64_t B, int32_t n, int64_t C) {
  if (check_shape(B, n, C) != MHC_OK || B == 0) return 0;
  return coeffs_ws_bytes(B, n, C, kPhi32);
}

int mhc_coeffs_phi32(int64_t B, int32_t n, int64_t C, const void *X_t, const float *phi,
                     float alpha_pre, float alpha_post, float alpha_res, const float *b_pre,
                     const float *b_post, const float *b_res, float *logits, float *r, float *H,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return coeffs_impl(kPhi32, B, n, C, X_t, phi, alpha_pre, alpha_post, alpha_res, b_pre, b_post,
                     b_res, logits, r, H, workspace, workspace_bytes, stream);
}

size_t mhc_post_res_coeffs_phi32_workspace_size(int64_t B, int32_t n, int64_t C) {
  return post_res_coeffs_ws_bytes(B, n, C, kPhi32);
}

int mhc_post_res_coeffs_phi32(int64_t B, int32_t n, int64_t C, const void *X_t, const void *F_out,
                              const float *H, void *X_next, const float *phi_next, float alpha_pre,
                              float alpha_post, float alpha_res, const float *b_pre,
                              const float *b_post, const float *b_res, float *logits_next,
                              float *r_next, float *H_next, void *workspace, size_t workspace_bytes,
                              void *stream) {
  return post_res_coeffs_impl(kPhi32, B, n, C, X_t, F_out, H, X_next, phi_next, alpha_pre,
                              alpha_post, alpha_res, b_pre, b_post, b_res, logits_next, r_next,
                              H_next, workspace, workspace_bytes, stream);
}

int mhc_lazy_prenorm_gemm(int64_t M, int64_t N, int64_t K, const void *A, const void *W,
                          float eps, void *C, float *rstd, void *stream) {
  if (M < 0 || N < 1 || K < 1) return MHC_ERR_INVALID_ARG;
  if (K % 8 != 0 || N % 8 != 0) return MHC_ERR_UNSUPPORTED;
  constexpr int64_t kMaxDim = (int64_t(1) << 31) - 256;
  constexpr int64_t kMaxLpnK = int64_t(1) << 22;  // 32-bit in-tile byte offsets
  if (M > kMaxDim || N > kMaxDim || K > kMaxLpnK ||
      (M > 0 && (M * K > kMaxElems || N * K > kMaxElems || M * N > kMaxElems)))
    return MHC_ERR_UNSUPPORTED;
  if (M == 0) return MHC_OK;
  if (!A || !W || !C) return MHC_ERR_INVALID_ARG;
  if (!aligned(A, 16) || !aligned(W, 16) || !aligned(C, 16) || (rstd && !aligned(rstd, 4)))
    return MHC_ERR_UNSUPPORTED;
  const Span sa = span(A, (size_t)(M * K * 2)), sw = span(W, (size_t)(N * K * 2));
  const Span sc = span(C, (size_t)(M * N * 2));
  if (overlaps(sc, sa) || overlaps(sc, sw)) return MHC_ERR_INVALID_ARG;
  if (rstd) {
    const Span sr = span(rstd, (size_t)M * 4);
    if (overlaps(sr, sa) || overlaps(sr, sw) || overlaps(sr, sc)) return MHC_ERR_INVALID_ARG;
  }
  return from_hip(mhc::launch_lazy_prenorm_gemm(M, N, K, A, W, eps, C, rstd,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
