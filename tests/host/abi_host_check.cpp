// Host-only check of libmhc's C ABI layer, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (the device code is built
// without them; no check here launches a kernel where a device is visible).
//
// Drives every argument-validation branch of the entry points in
// include/mhc.h with fake device addresses (never dereferenced on the host),
// extreme sizes (to expose overflow in the size arithmetic), the tuning
// keys, the one-pass grid arithmetic, and -- on a host with no HIP device --
// calls that pass validation, which must report MHC_ERR_HIP.  Exits non-zero
// on the first failed check; the sanitizers abort on any error they find.
#include "mhc.h"
#include "mhc_launch.h"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

namespace {

int g_checks = 0;

#define CHECK(cond)                                                                 \
  do {                                                                              \
    ++g_checks;                                                                     \
    if (!(cond)) {                                                                  \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      std::exit(1);                                                                 \
    }                                                                               \
  } while (0)

// Fake, 16-byte aligned device addresses far apart (never dereferenced).
void *addr(int k) { return reinterpret_cast<void *>(uintptr_t(1) << 44 | (uintptr_t)k << 38); }
float *faddr(int k) { return static_cast<float *>(addr(k)); }

int coeffs(int64_t B, int32_t n, int64_t C, size_t ws, int skip = -1, uintptr_t misalign = 0) {
  void *p[10];
  for (int k = 0; k < 10; ++k) p[k] = k == skip ? nullptr : addr(k);
  if (misalign) p[0] = static_cast<char *>(p[0]) + misalign;
  return mhc_coeffs(B, n, C, p[0], p[1], 0.01f, 0.01f, 0.01f, (float *)p[2], (float *)p[3], (float *)p[4],
                    (float *)p[5], (float *)p[6], (float *)p[7], p[8], ws, nullptr);
}

int fused_pre(int64_t B, int32_t n, int64_t C, size_t ws, int skip = -1) {
  void *p[14];
  for (int k = 0; k < 14; ++k) p[k] = k == skip ? nullptr : addr(k);
  return mhc_post_res_coeffs_pre(B, n, C, p[0], p[1], (float *)p[2], p[3], p[4], 0.01f, 0.01f, 0.01f,
                                 (float *)p[5], (float *)p[6], (float *)p[7], (float *)p[8], (float *)p[9],
                                 (float *)p[10], p[11], p[12], ws, nullptr);
}

}  // namespace

int main(int argc, char **argv) {
  const bool no_device = argc > 1 && argv[1][0] == '1';

  // Status strings.
  for (int s = 0; s <= 5; ++s) CHECK(mhc_status_string(s) != nullptr && mhc_status_string(s)[0] == 'M');
  CHECK(mhc_status_string(-7) != nullptr && mhc_status_string(1 << 30) != nullptr);

  // Workspace-size and split functions over ordinary and extreme shapes.
  const int64_t Bs[] = {0, 1, 17, 64, 256, 257, 4096, 16384, int64_t(1) << 31, INT64_MAX, -1, INT64_MIN};
  const int32_t ns[] = {1, 2, 3, 4, 8, 0, -4, INT32_MAX, INT32_MIN};
  const int64_t Cs[] = {8,        16,   24, 32, 40, 512, 1024, 7168, 8704, int64_t(1) << 30, int64_t(1) << 62,
                        INT64_MAX - 7, INT64_MAX, 0, -8};
  for (int64_t B : Bs)
    for (int32_t n : ns)
      for (int64_t C : Cs) {
        const size_t a = mhc_coeffs_workspace_size(B, n, C);
        const size_t b = mhc_post_res_coeffs_workspace_size(B, n, C);
        const size_t c = mhc_post_res_coeffs_pre_workspace_size(B, n, C);
        const size_t d = mhc_coeffs_fp8_workspace_size(B, n, C);
        const size_t e = mhc_post_res_coeffs_pre_fp8_workspace_size(B, n, C);
        const size_t f = mhc_coeffs_phi32_workspace_size(B, n, C);
        const size_t g = mhc_post_res_coeffs_phi32_workspace_size(B, n, C);
        (void)mhc_post_res_coeffs_fp8_workspace_size(B, n, C);
        const int32_t s = mhc_coeffs_split_k(B, n, C);
        const bool valid = B > 0 && (n == 1 || n == 2 || n == 4 || n == 8) && C > 0 && C % 8 == 0 &&
                           B < (int64_t(1) << 31) && C <= (int64_t(1) << 30) / n;
        if (!valid) CHECK(a == 0 && b == 0 && c == 0 && d == 0 && e == 0 && f == 0 && g == 0 && s == 0);
        if (valid && B <= ((int64_t(1) << 40) - 1) / ((int64_t)n * C)) CHECK(a > 0 && s >= 1 && f > 0);
        (void)mhc_post_res_coeffs_pre_one_pass(B, n, C);
        (void)mhc_post_res_coeffs_pre_fp8_one_pass(B, n, C);
      }

  // mhc_coeffs validation.
  const size_t ws = mhc_coeffs_workspace_size(64, 4, 256);
  CHECK(ws > 0);
  CHECK(coeffs(0, 4, 256, 0, 0) == MHC_OK);                       // B == 0: nothing checked beyond the shape
  CHECK(coeffs(-1, 4, 256, ws) == MHC_ERR_INVALID_ARG);
  CHECK(coeffs(64, 0, 256, ws) == MHC_ERR_INVALID_ARG);
  CHECK(coeffs(64, 3, 256, ws) == MHC_ERR_UNSUPPORTED);
  CHECK(coeffs(64, 4, 252, ws) == MHC_ERR_UNSUPPORTED);
  CHECK(coeffs(INT64_MAX, 4, 256, ws) == MHC_ERR_UNSUPPORTED);
  CHECK(coeffs(64, 4, INT64_MAX - 7, ws) == MHC_ERR_UNSUPPORTED);
  for (int k = 0; k < 9; ++k) CHECK(coeffs(64, 4, 256, ws, k) == MHC_ERR_INVALID_ARG);
  CHECK(coeffs(64, 4, 256, ws, -1, 8) == MHC_ERR_UNSUPPORTED);   // X_t misaligned
  CHECK(coeffs(64, 4, 256, ws - 1) == MHC_ERR_WORKSPACE);
  {
    // output overlapping an input
    float *x = faddr(0);
    CHECK(mhc_coeffs(64, 4, 256, x, addr(1), 0.01f, 0.01f, 0.01f, faddr(2), faddr(3), faddr(4), x + 64,
                     faddr(6), faddr(7), addr(8), ws, nullptr) == MHC_ERR_INVALID_ARG);
  }

  // pre / post_res validation (bf16 and E4M3).
  CHECK(mhc_pre(0, 4, 64, nullptr, nullptr, nullptr, nullptr) == MHC_OK);
  CHECK(mhc_pre(16, 4, 64, addr(0), faddr(1), nullptr, nullptr) == MHC_ERR_INVALID_ARG);
  CHECK(mhc_pre(16, 4, 64, addr(0), faddr(1), addr(0), nullptr) == MHC_ERR_INVALID_ARG);  // F_pre overlaps X_t
  CHECK(mhc_pre_fp8(16, 4, 24, addr(0), faddr(1), addr(2), nullptr) == MHC_ERR_UNSUPPORTED);
  CHECK(mhc_post_res(16, 4, 64, addr(0), addr(1), faddr(2), addr(0), nullptr) == MHC_ERR_INVALID_ARG);
  CHECK(mhc_post_res_fp8(16, 4, 40, addr(0), addr(1), faddr(2), addr(3), nullptr) == MHC_ERR_UNSUPPORTED);
  CHECK(mhc_post_res(16, 4, 64, static_cast<char *>(addr(0)) + 2, addr(1), faddr(2), addr(3), nullptr) ==
        MHC_ERR_UNSUPPORTED);

  // The one-pass call and its check.
  const size_t wsp = mhc_post_res_coeffs_pre_workspace_size(16, 4, 64);
  CHECK(wsp > 0);
  CHECK(fused_pre(0, 4, 64, 0, 0) == MHC_OK);
  CHECK(fused_pre(16, 4, 48, wsp) == MHC_ERR_UNSUPPORTED);      // C % 32 != 0
  for (int k = 0; k < 13; ++k) CHECK(fused_pre(16, 4, 64, wsp, k) == MHC_ERR_INVALID_ARG);
  CHECK(fused_pre(16, 4, 64, wsp - 1) == MHC_ERR_WORKSPACE);
  CHECK(mhc_post_res_coeffs_pre_check(64, 4, 7168, 0, addr(0), 1 << 20, nullptr) == MHC_OK);  // two calls
  CHECK(mhc_post_res_coeffs_pre_check(16384, 3, 7168, 0, addr(0), 1 << 20, nullptr) == MHC_ERR_UNSUPPORTED);
  const size_t wbig = mhc_post_res_coeffs_pre_workspace_size(16384, 4, 7168);
  CHECK(mhc_post_res_coeffs_pre_check(16384, 4, 7168, 0, addr(0), wbig - 1, nullptr) == MHC_ERR_WORKSPACE);
  CHECK(mhc_post_res_coeffs_pre_check(16384, 4, 7168, 1, nullptr, 0, nullptr) == MHC_ERR_INVALID_ARG);

  // The allocation-free call: validation and its size limit (nothing launched).
  {
    void *p[13];
    for (int k = 0; k < 13; ++k) p[k] = addr(k);
    auto na = [&](int64_t B, int32_t n, int64_t C) {
      return mhc_post_res_coeffs_pre_noalloc(B, n, C, p[0], p[1], (float *)p[2], p[3], p[4], 0.01f, 0.01f,
                                             0.01f, (float *)p[5], (float *)p[6], (float *)p[7], (float *)p[8],
                                             (float *)p[9], (float *)p[10], p[11], nullptr);
    };
    CHECK(na(0, 4, 64) == MHC_OK);
    CHECK(na(16, 3, 64) == MHC_ERR_UNSUPPORTED);
    CHECK(na(16, 4, 48) == MHC_ERR_UNSUPPORTED);
    CHECK(na(-3, 4, 64) == MHC_ERR_INVALID_ARG);
    CHECK(mhc_post_res_coeffs_pre_workspace_size(65536, 4, 7168) > MHC_NOALLOC_SCRATCH_BYTES);
    CHECK(na(65536, 4, 7168) == MHC_ERR_WORKSPACE);
  }

  // Lazy Pre-Norm GEMM validation.
  CHECK(mhc_lazy_prenorm_gemm(0, 64, 64, nullptr, nullptr, 1e-5f, nullptr, nullptr, nullptr) == MHC_OK);
  CHECK(mhc_lazy_prenorm_gemm(-1, 64, 64, addr(0), addr(1), 1e-5f, addr(2), nullptr, nullptr) ==
        MHC_ERR_INVALID_ARG);
  CHECK(mhc_lazy_prenorm_gemm(64, 60, 64, addr(0), addr(1), 1e-5f, addr(2), nullptr, nullptr) ==
        MHC_ERR_UNSUPPORTED);
  CHECK(mhc_lazy_prenorm_gemm(64, 64, (int64_t(1) << 22) + 8, addr(0), addr(1), 1e-5f, addr(2), nullptr,
                              nullptr) == MHC_ERR_UNSUPPORTED);
  CHECK(mhc_lazy_prenorm_gemm(INT64_MAX, INT64_MAX, INT64_MAX - 7, addr(0), addr(1), 1e-5f, addr(2), nullptr,
                              nullptr) == MHC_ERR_UNSUPPORTED);
  CHECK(mhc_lazy_prenorm_gemm(64, 64, 64, addr(0), addr(1), 1e-5f, addr(0), nullptr, nullptr) ==
        MHC_ERR_INVALID_ARG);

  // Tuning keys.
  CHECK(mhc_tuning_set(nullptr, 1) == MHC_ERR_INVALID_ARG);
  CHECK(mhc_tuning_set("MHC_NOPE", 1) == MHC_ERR_INVALID_ARG);
  const int32_t s0 = mhc_coeffs_split_k(8192, 8, 4224);  // the split-K product (the default at n = 8 above C = 4096)
  CHECK(mhc_tuning_set("MHC_SPLIT_K", 5) == MHC_OK && mhc_coeffs_split_k(8192, 8, 4224) == 5);
  CHECK(mhc_tuning_set("MHC_SPLIT_K", INT64_MAX) == MHC_OK && mhc_coeffs_split_k(8192, 8, 4224) >= 1);
  CHECK(mhc_tuning_set("MHC_FUSED_PRE", 0) == MHC_OK && !mhc_post_res_coeffs_pre_one_pass(16384, 4, 7168));
  for (const char *k : {"MHC_SMALL_MAX_B", "MHC_GEMM_ALGO", "MHC_GEMM_WGS", "MHC_GEMM_MB", "MHC_FUSED_N8",
                        "MHC_FUSED_FP8", "MHC_FUSED_FIXED", "MHC_FUSED_SPU", "MHC_FUSED_WGS", "MHC_LPN_ALGO",
                        "MHC_GEMM_KC", "MHC_GEMM_STAGES"}) {
    CHECK(mhc_tuning_set(k, INT64_MAX) == MHC_OK);
    for (int64_t B : {int64_t(64), int64_t(4096), int64_t(16384)})
      for (int32_t n : {1, 4, 8}) {
        (void)mhc_coeffs_workspace_size(B, n, 7168);
        (void)mhc_post_res_coeffs_pre_workspace_size(B, n, 4096);
      }
    CHECK(mhc_tuning_set(k, -5) == MHC_OK);
  }
  mhc_tuning_reset();
  CHECK(mhc_coeffs_split_k(8192, 8, 4224) == s0 && mhc_post_res_coeffs_pre_one_pass(16384, 4, 7168));

  // The one-pass grid: whole row tiles per round within what is resident.
  CHECK(mhc::pre_mode_grid(1024 * 14, 14, 256, -1) == 252);
  CHECK(mhc::pre_mode_grid(1024 * 14, 14, 256, 100) == 98);
  CHECK(mhc::pre_mode_grid(2 * 14, 14, 256, -1) == 28);     // fewer units than workgroups
  CHECK(mhc::pre_mode_grid(1024 * 14, 14, 13, -1) == 0);    // one row tile's slices do not fit
  CHECK(mhc::pre_mode_grid(1024 * 14, 14, 14, -1) == 14);
  CHECK(mhc::pre_mode_grid(1024 * 14, 14, 0, -1) == 0);
  CHECK(mhc::pre_mode_grid(0, 14, 256, -1) == 0);
  CHECK(mhc::pre_mode_grid(1024 * 16, 16, 256, -1) == 256);
  CHECK(mhc::pre_mode_grid(1024, 1, 200, 7) == 7);
  for (int64_t S = 1; S <= 16; ++S)
    for (int64_t R : {int64_t(0), int64_t(1), int64_t(63), int64_t(255), int64_t(256), int64_t(1) << 40})
      for (int64_t U : {int64_t(0), S, 7 * S, 1000 * S}) {
        const int64_t G = mhc::pre_mode_grid(U, S, R, -1);
        CHECK(G == 0 || (G % S == 0 && G <= R && G <= U && G >= S));
      }

  // No HIP device: calls that pass validation cannot launch.
  if (no_device) {
    CHECK(mhc_pre(16, 4, 64, addr(0), faddr(1), addr(2), nullptr) == MHC_ERR_HIP);
    CHECK(coeffs(64, 4, 256, ws) == MHC_ERR_HIP);
    CHECK(fused_pre(16384, 4, 7168, wbig) == MHC_ERR_HIP);
    CHECK(mhc_post_res_coeffs_pre_check(16384, 4, 7168, 0, addr(0), wbig, nullptr) == MHC_ERR_HIP);
    CHECK(mhc_lazy_prenorm_gemm(64, 64, 64, addr(0), addr(1), 1e-5f, addr(2), nullptr, nullptr) == MHC_ERR_HIP);
  }
  std::printf("abi_host_check: %d checks passed%s\n", g_checks, no_device ? " (no-device calls included)" : "");
  return 0;
}
