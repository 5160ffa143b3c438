// Host-side launch interface between the C-ABI layer (mhc_abi.hip) and the
// kernel translation units.  Arguments are validated by the caller; these
// functions only pick launch shapes and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

// Route and launch-shape overrides for tests and tuning (mhc_tuning_set in
// mhc.h).  Every key starts unset (-1), which selects the measured default;
// the library never reads the environment, so nothing outside an explicit
// mhc_tuning_set call changes which kernels run or in what order they sum.
enum TuneKey : int {
  kTuneSmallMaxB = 0,  // rows up to which the one-launch small-B kernel runs (0: never)
  kTuneGemmAlgo,       // 0: register-path product; 2: persistent product kernel
  kTuneSplitK,         // K-slices of the split-K product (> 0)
  kTuneGemmWgs,        // target workgroup count of the split-K product (> 0)
  kTuneGemmMb,         // 16-row blocks per wave of the E4M3 split-K product (1 or 2)
  kTuneFusedN8,        // > 0: the fused kernel also at n = 8
  kTuneFusedFp8,       // 0: E4M3 fused call as apply + product; > 0: fused kernel
  kTuneFusedFixed,     // 0 / 1: fused kernel's fixed-slice layout off / on
  kTuneFusedSpu,       // 512-channel steps per unit of the fused kernel (> 0)
  kTuneFusedWgs,       // workgroups of the fused kernel (> 0; never above the resident count)
  kTuneFusedPre,       // 0: mhc_post_res_coeffs_pre(_fp8) as two calls
  kTuneLpnAlgo,        // Lazy Pre-Norm GEMM: 0 eight-wave kernel, 1 four-wave kernel
  kTuneGemmKc,         // 128: the bf16 split-K product in 128-k chunks (with kTuneGemmStages)
  kTuneGemmStages,     // 5 or 6: its ring depth
  kTuneGemmWaves,      // 4 or 8: wavefronts per workgroup of the LDS-staged split-K product
  kTuneGemmXreg,       // 2: bf16 split-K product with X and phi through two register sets (n = 4, 8)
  kTuneApplySmall,     // 0: small-B bf16 mhc_post_res_coeffs as the apply kernel, then coeffs_small
  kTunePass8Sets,      // 1 or 2: register sets of loads of the n = 8 pass with the hand-off
  kTunePass8Pre,       // 1: mhc_post_res_coeffs_pre and mhc_coeffs_pre at n = 8 in one pass (default: two calls)
  kTuneCount
};
// Current value of a key; -1 when unset.
int64_t tune(TuneKey k);

// Compute units of the current device (queried once per device id).
int device_cus();

// Split-K plan of the fused product + sum-of-squares pass.
//
// Workspace layout (bytes from the start of the caller's workspace):
//   [0, partial_bytes)                 fp32 partials [split, B, N+1]
//   [phip_offset, +phip_bytes)         packed phi (algo 1 only)
//   [zero_offset, +256)                zero block (algo 1 only)
struct GemmPlan {
  int algo;           // 0: MFMA A operands loaded from global memory; 1: X staged through LDS
  int mb;             // 16-row MFMA blocks per wavefront (rows per workgroup = 16 * mb * waves)
  int waves;          // wavefronts per workgroup: 4, or 8 (algo 1 only)
  int xreg;           // 2: X and phi through two register sets (algo 1, bf16, n = 4 or 8, W = 8)
  int kc;             // K elements per chunk
  int stages;         // LDS ring depth (algo 1)
  int xb;             // bytes per X element: 2 (bf16) or 1 (E4M3, algo 1 only)
  int phi_parts;      // 1: bf16 phi; 2: fp32 phi packed as hi + lo bf16 parts (algo 1 only)
  int split;          // S: number of K-slices (partials in the workspace)
  int64_t kslice;     // K elements per slice (multiple of kc)
  int64_t row_tiles;  // workgroups along B
  size_t partial_bytes, phip_offset, phip_bytes, zero_offset, total_bytes;
};

GemmPlan plan_gemm(int64_t B, int n, int64_t C, bool fp8_x = false, bool phi32 = false);
// Plan with explicit kernel, rows-per-wave blocks, chunk size, ring depth and
// target workgroup count.
GemmPlan plan_gemm_custom(int64_t B, int n, int64_t C, int algo, int mb, int kc, int stages,
                          int64_t target_wgs, int waves = 4);
size_t gemm_workspace_bytes(const GemmPlan &p, int64_t B, int n);

template <int NS, int W, int KC, int D>
hipError_t launch_gemm_xreg_typed(const GemmPlan &p, int64_t B, int64_t C, const void *X, const void *phi,
                                  void *ws_base, hipStream_t st);

template <int NS, int MB, int KC, int STAGES, int XB, int P2, int W = 4>
hipError_t launch_gemm_lds_typed(const GemmPlan &p, int64_t B, int64_t C, const void *X,
                                 const void *phi, void *ws_base, hipStream_t st);

hipError_t launch_gemm_rms(const GemmPlan &p, int n, int64_t B, int64_t C,
                           const void *X, const void *phi, float *ws, hipStream_t st);

// phi [K, N] -> packed MFMA B operands ([ksteps][NB][64 lanes][8] bf16, zero
// past K and past N) plus a 256-byte zero block.  The same launch zero-fills
// clear[0, clear_bytes) when clear is given (clear_bytes a multiple of 16).
hipError_t launch_pack_phi(int n, int64_t K, int64_t ksteps, const void *phi, void *phip,
                           void *zero, hipStream_t st, void *clear = nullptr,
                           size_t clear_bytes = 0);
// fp32 phi [K, N] -> per 32-k step the NB blocks of phi_hi = bf16(phi), then
// the NB blocks of phi_lo = bf16(phi - phi_hi) (layout as above), plus the
// zero block.
hipError_t launch_pack_phi32(int n, int64_t K, int64_t ksteps, const void *phi, void *phip,
                             void *zero, hipStream_t st);

// Fused apply of this layer + coefficient product of the next (one pass).
//
// Workspace layout: [0, partial_bytes) fp32 partials [split, B, N+1];
// [phip_offset, +phip_bytes) packed phi of the next layer; [zero_offset, +256).
//
// The pre-mix mode (pre = true in the plan) adds, after the zero block:
// [rec_offset, +rec_bytes) hand-off records [B, split, PW] (4 bytes each,
// PW = n+1 rounded up to even) and [flag_offset, +16) the give-up word (a
// uint32, non-zero once a wait for records gave up); both zero-filled by the
// launch before the kernel runs.
struct FusedPlan {
  int split;          // channel slices (K-slices of n*cw)
  int cw;             // channels per slice (multiple of 512)
  int64_t row_tiles;  // 16-row tiles
  int64_t ksteps;     // packed phi 32-k steps
  bool pre;           // pre-mix mode layout
  bool fixed;         // fixed-slice layout: one step per unit, whole row tiles per round
  size_t partial_bytes, dummy_offset, dummy_bytes, phip_offset, phip_bytes, zero_offset;
  size_t rec_offset, rec_bytes, flag_offset, total_bytes;
};
// prefer_fixed: take the fixed-slice layout where it fits (n <= 4) unless
// MHC_FUSED_FIXED=0; without it, only with MHC_FUSED_FIXED=1.  The pre-mix
// mode always takes it.  Measured on MI355X (n=4, C=7168, B=16384, chained
// layers): the E4M3 apply and both product-only modes run faster in it; the
// bf16 apply after mhc_pre runs slower (393 vs 381 us).
FusedPlan plan_post_res_next(int64_t B, int n, int64_t C, bool pre = false, bool prefer_fixed = false);
// Whether the fixed-slice layout fits (n <= 4, one workgroup per slice at
// least, phi itself addressable by 32-bit offsets).
bool fixed_layout_fits(int n, int64_t C);
// What the persistent kernel of mhc_post_res_fused.hip does per step.
enum FusedMode : int {
  kFusedApplyBf16 = 0,     // bf16 X_t, F_out -> bf16 X_next, plus X_next . phi_next
  kFusedApplyFp8 = 1,      // E4M3 X_t, F_out -> E4M3 X_next, plus X_next . phi_next
  kFusedCoeffsFp8 = 2,     // X . phi only, X in E4M3
  kFusedCoeffsBf16 = 3,    // X . phi only, X in bf16
  kFusedApplyPreBf16 = 4,  // kFusedApplyBf16, plus the next layer's F_pre (n <= 4)
  kFusedApplyPreFp8 = 5,   // kFusedApplyFp8, plus the next layer's F_pre in E4M3 (n <= 4)
  kFusedCoeffsPreBf16 = 6, // kFusedCoeffsBf16, plus this layer's F_pre (n <= 4)
  kFusedCoeffsPreFp8 = 7,  // kFusedCoeffsFp8, plus this layer's F_pre in E4M3 (n <= 4)
};
constexpr bool is_pre_mode(int mode) {
  return mode == kFusedApplyPreBf16 || mode == kFusedApplyPreFp8 || mode == kFusedCoeffsPreBf16 ||
         mode == kFusedCoeffsPreFp8;
}
// Kernel-side arguments of the pre-mix mode.  Its stores of partials,
// records and F_pre, and its record loads, go through buffer resources, so a
// store without a target is given an offset past the buffer and dropped by
// the hardware: no dummy area, no branch, no memory traffic.
struct PreArgs {
  void *F_pre;                    // bf16 or E4M3 [B, C]
  uint32_t *rec;                  // records [B, split, PW]: fp32 bits, 0 = not yet written
  uint32_t rec_bytes;             // split * B * PW * 4 (< 2^31); PW = n+1 rounded up to even
  uint32_t partial_bytes;         // split * B * (N+1) * 4 (< 2^31)
  uint32_t phip_bytes;            // packed phi (< 2^31)
  const uint16_t *phi;            // the fixed-slice layout: phi [K, N] itself (gathered once per run)
  uint32_t phi_bytes;             // K * N * 2 (< 2^31)
  const float *b_pre;             // fp32 [n]
  float alpha_pre, inv_k;         // alpha_pre; 1 / (n C)
  uint32_t *giveup;               // set non-zero by a wave whose wait for records gave up
};
// Whether the pre-mix mode can run this shape: n <= 4, at most 16
// 512-channel steps per row (the record gather), a grid of whole row tiles
// (a multiple of S workgroups) that fits the device, and partials and
// records addressable by 32-bit buffer offsets.
bool pre_mode_fits(int64_t B, int n, int64_t C);
// Workgroups of the pre-mix kernel (n, mode) that can be resident at
// once for launches on `st`: the per-CU occupancy the runtime reports for the
// kernel times the compute units the stream may use (its CU mask).  Cached
// per device and kernel, except the mask, which is read per call.
int64_t pre_mode_resident(int n, int mode, hipStream_t st);
// Grid of the pre-mix mode: whole row tiles per round (a multiple of
// `split`), at most `resident` workgroups (and at most `wgs_cap` when that is
// positive), no more than the `units` there are; 0 when not even one row
// tile's `split` workgroups can be resident together (the mode must not run).
int64_t pre_mode_grid(int64_t units, int64_t split, int64_t resident, int64_t wgs_cap);
// Compute units a launch on `st` may use: the device's, or the stream's CU
// mask where it has one.
int64_t stream_cus(hipStream_t st);
// pre_out: F_pre (bf16 or E4M3 [B, C], the element type of the mode), the
// next layer's b_pre / alpha_pre and the grid (pre_mode_grid) for the
// pre-mix modes, else null.
struct PreOut {
  void *F_pre;
  const float *b_pre;
  float alpha_pre;
  int64_t grid;
};
hipError_t launch_post_res_next(const FusedPlan &p, int n, int mode, int64_t B, int64_t C,
                                const void *X, const void *F, const float *H, void *Y,
                                const void *phi_next, void *ws_base, hipStream_t st,
                                const PreOut *pre_out = nullptr);

// The n = 8 pass (mhc_onepass8.hip): bf16, one workgroup per 128-channel
// slice of all 8 streams and row tile, phi held in registers.  apply: X_t,
// F_out, H -> X_next (mhc_post_res's bits) and the next layer's partials;
// otherwise the partials of X_t itself.  With plan.pre also the records and
// F_pre (pre_out).  Workspace: the FusedPlan of plan_onepass8 (partials
// [S, B, 81]; with pre, records [B, 9, S] and the give-up word, zero-filled
// by the launch).  The combine is launch_coeff_sinkhorn(..., tree = true).
constexpr int kMaxSlices8 = 32;  // slices per row: C <= 4096
bool onepass8_fits(int64_t B, int64_t C);
FusedPlan plan_onepass8(int64_t B, int64_t C, bool pre);
// Workgroups that can be resident at once for launches on `st`.
int64_t onepass8_resident(bool apply, bool pre, hipStream_t st);
// grid: a multiple of plan.split, at most the row tiles times the split, all
// resident (pre_mode_grid with onepass8_resident).
hipError_t launch_onepass8(const FusedPlan &p, bool apply, int64_t B, int64_t C, const void *X,
                           const void *F, const float *H, void *Y, const void *phi, void *ws_base,
                           int64_t grid, hipStream_t st, const PreOut *pre_out);

// Single-slice layer calls in one kernel (mhc_layer_small.hip): the one-pass
// mhc_post_res_coeffs_pre / mhc_coeffs_pre in bf16 for n in {1, 2, 4} at the
// small-B sizes of mhc_coeffs when a row's n*C channels fit 1024 (C % 8 == 0).
// One workgroup per 16-row tile; no workspace.
bool layer_small_fits(int64_t B, int n, int64_t C);
// apply: mhc_post_res_coeffs_pre (X = X_t, F = F_out, H, Y = X_next);
// otherwise mhc_coeffs_pre (X = X_t; F, H, Y unused).
hipError_t launch_layer_small(int n, bool apply, int64_t B, int64_t C, const void *X, const void *F,
                              const float *H, void *Y, const void *phi, float ap, float aq, float ar,
                              const float *bp, const float *bq, const float *br, float *logits, float *r,
                              float *Hn, void *F_pre, hipStream_t st);

// Zero-fill [p, p + bytes) (bytes a multiple of 16, p 16-byte aligned) with a
// small kernel (no memset node if the caller captures a graph).
hipError_t launch_zero(void *p, size_t bytes, hipStream_t st);

// Lazy Pre-Norm GEMM C = rmsnorm(A) W^T (mhc_lazy_prenorm.hip).
hipError_t launch_lazy_prenorm_gemm(int64_t M, int64_t N, int64_t K, const void *A, const void *W,
                                    float eps, void *C, float *rstd, hipStream_t st);

// FP8 (E4M3) streaming kernels (mhc_stream_fp8.hip).
hipError_t launch_pre_fp8(int n, int64_t B, int64_t C, const void *X, const float *H,
                          void *F_pre, hipStream_t st);
hipError_t launch_post_res_fp8(int n, int64_t B, int64_t C, const void *X, const void *F_out,
                               const float *H, void *X_next, hipStream_t st);

// Small-B (decode) path of mhc_coeffs: product, split-K reduction and finish
// in one launch (mhc_coeffs_small.hip).
//
// Workspace layout: [0, partial_bytes) fp32 partials [split, B, N+1];
// [ctr_offset, +8 * row_tiles * split) one 64-bit arrival flag per 16-row
// tile and K-slice (any initial contents).
template <int NS>
constexpr int kSmallKSlice() { return NS >= 8 ? 256 : 1024; }  // K per slice: phi slice <= 48 KiB of LDS
constexpr int64_t kSmallMaxB = 256;     // rows up to which mhc_coeffs takes this path
constexpr int64_t kSmallMaxSplit = 64;  // ... and K-slices up to which
// Slices whose partials a small-B finisher loads at once (ept sums per thread).
constexpr int combine_batch(int ept) { return ept <= 2 ? 32 : 16; }
struct SmallPlan {
  int split;
  int64_t kslice, row_tiles;
  size_t partial_bytes, ctr_offset, total_bytes;
};
SmallPlan plan_coeffs_small(int64_t B, int n, int64_t C);
bool use_coeffs_small(int64_t B, int n, int64_t C);
// fp8_x: X holds E4M3 values (widened exactly to bf16 for the product).
hipError_t launch_coeffs_small(const SmallPlan &p, int n, bool fp8_x, int64_t B, int64_t C,
                               const void *X, const void *phi, float alpha_pre, float alpha_post,
                               float alpha_res, const float *b_pre, const float *b_post,
                               const float *b_res, float *logits, float *r, float *H, void *ws,
                               hipStream_t st,
                               bool phi32 = false);

// mhc_post_res_coeffs at the small-B sizes in one kernel (mhc_layer_small.hip):
// bf16, n in {1, 2, 4}, C % 8 == 0; the apply, then split-K over channel
// ranges of all n streams with the last workgroup of a tile to arrive
// finishing it.  Workspace and flags as coeffs_small (plan_coeffs_small gives
// the same slice count, ceil(n*C / 1024)).
bool apply_coeffs_small_fits(int64_t B, int n, int64_t C);
hipError_t launch_apply_coeffs_small(const SmallPlan &p, int n, int64_t B, int64_t C, const void *X,
                                     const void *F, const float *H, void *Y, const void *phi, float ap, float aq,
                                     float ar, const float *bp, const float *bq, const float *br, float *logits,
                                     float *r, float *Hn, void *ws, hipStream_t st);
// Process-wide 64-bit call epoch of the small-B arrival flags (never 0).
unsigned long long next_call_epoch();

// tree: add the split partials as the balanced tree over 16 slots (split <=
// 16, n <= 4), the order of the fused kernel's pre-mix mode, or at n = 8 over
// 32 slots (split <= 32: two 16-slot trees, then their sum), the order of the
// n = 8 pass.
hipError_t launch_coeff_sinkhorn(int n, int64_t B, int64_t C, int split, const float *ws,
                                 float alpha_pre, float alpha_post, float alpha_res,
                                 const float *b_pre, const float *b_post, const float *b_res,
                                 float *logits, float *r, float *H, hipStream_t st,
                                 bool tree = false);

hipError_t launch_pre(int n, int64_t B, int64_t C, const void *X, const float *H,
                      void *F_pre, hipStream_t st);

hipError_t launch_post_res(int n, int64_t B, int64_t C, const void *X, const void *F_out,
                           const float *H, void *X_next, hipStream_t st);

}  // namespace mhc
