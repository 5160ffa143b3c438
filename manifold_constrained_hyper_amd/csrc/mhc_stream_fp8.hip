// Streaming kernels of the FP8 residual-stream variant: X_t, F_out, F_pre and
// X_next in E4M3 (unscaled, the OCP "fn" encoding), coefficients in fp32.
//
// [mHC-cutile] (page "mHC 算法分析 & cutile 高效实现") runs its first
// benchmark with every tensor in torch.float8_e4m3fn; the arithmetic is that of
// section 2.5 (and the fused apply of section 3.4) as in mhc_stream.hip: fp32
// accumulation of the widened inputs, one rounding to E4M3 at the end (to
// nearest even, saturating at +-448).  At n = 4 the post/res mix runs on the
// matrix core (mix4_pair, mhc_device.h: H carried to 2^-17 relative as two
// bf16 parts, products exact, fp32 sums), as in the fused kernel's E4M3
// apply, so both write the same bits.
//
// Layout of the work as in mhc_stream.hip: one wavefront per (row, chunk)
// task, a chunk being 64 consecutive 16-byte vectors of 16 E4M3 channels, so
// every load/store instruction of a wave touches 1 KiB of contiguous memory
// per stream; the row's coefficients come by scalar loads; all loads of a task
// are issued before any arithmetic.
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float (&v)[4]) {
  const f32x2 a = fp8_lo2(w), b = fp8_hi2(w);
  v[0] = a[0];
  v[1] = a[1];
  v[2] = b[0];
  v[3] = b[1];
}

// F_pre[row, c] = sum_i H_pre[row, i] * X[row, i*C + c]
template <int NS>
__global__ __launch_bounds__(64) void pre_fp8_kernel(const uint8_t *__restrict__ X,
                                                     const float *__restrict__ H,
                                                     uint8_t *__restrict__ F, uint32_t cvec,
                                                     uint32_t chunks_per_row, uint32_t tasks) {
  constexpr int N = NS * NS + 2 * NS;
  const uint32_t task = (uint32_t)uniform((int)blockIdx.x);
  if (task >= tasks) return;
  const uint32_t row = task / chunks_per_row;
  const uint32_t chunk = task - row * chunks_per_row;
  const float *h = H + (size_t)row * N;
  float hpre[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) hpre[i] = h[i];

  const uint8_t *xr = X + (size_t)row * NS * cvec * 16;
  uint8_t *fr = F + (size_t)row * cvec * 16;
  const uint32_t v = chunk * 64u + (threadIdx.x & 63u);
  if (v >= cvec) return;
  u32x4 xv[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j)
    xv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + ((size_t)j * cvec + v) * 16));
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      float x[4];
      fp8x4_to_f32(xv[j][w], x);
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] = fmaf(hpre[j], x[k], a[k]);
    }
    out[w] = pack_fp8x4(a[0], a[1], a[2], a[3]);
  }
  store16_plain(fr + (size_t)v * 16, out);
}

// X_next[row, i*C + c] = sum_j H_res[row, i, j] * X[row, j*C + c] + H_post[row, i] * F_out[row, c]
template <int NS>
__global__ __launch_bounds__(64) void post_res_fp8_kernel(const uint8_t *__restrict__ X,
                                                          const uint8_t *__restrict__ F,
                                                          const float *__restrict__ H,
                                                          uint8_t *__restrict__ Y, uint32_t cvec,
                                                          uint32_t chunks_per_row, uint32_t tasks) {
  constexpr int N = NS * NS + 2 * NS;
  const uint32_t task = (uint32_t)uniform((int)blockIdx.x);
  if (task >= tasks) return;
  const uint32_t row = task / chunks_per_row;
  const uint32_t chunk = task - row * chunks_per_row;
  const float *h = H + (size_t)row * N;
  float hpost[NS], hres[NS][NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    hpost[i] = h[NS + i];
#pragma unroll
    for (int j = 0; j < NS; ++j) hres[i][j] = h[2 * NS + i * NS + j];
  }

  const size_t xrow = (size_t)NS * cvec * 16;
  const uint8_t *xr = X + (size_t)row * xrow;
  const uint8_t *fr = F + (size_t)row * cvec * 16;
  uint8_t *yr = Y + (size_t)row * xrow;
  const uint32_t v_raw = chunk * 64u + (threadIdx.x & 63u);
  // At n = 4 the mix runs on the matrix core, whose 4x4x4 blocks take A rows
  // from four neighbouring lanes: every lane stays, lanes past the row
  // compute on its last vector and store nothing.
  if (NS != 4 && v_raw >= cvec) return;
  const uint32_t v = v_raw < cvec ? v_raw : cvec - 1;
  u32x4 xv[NS], fv;
#pragma unroll
  for (int j = 0; j < NS; ++j)
    xv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + ((size_t)j * cvec + v) * 16));
  fv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(fr + (size_t)v * 16));
  u32x4 out[NS];
  if constexpr (NS == 4) {
    // Row (lane & 3) of H_res and H_post[lane & 3] (per-lane loads; H is only
    // 4-byte aligned).
    const int i4 = threadIdx.x & 3;
    const float *hr = h + 2 * NS + i4 * NS;
    const Mix4A ma = mix4_a(hr[0], hr[1], hr[2], hr[3], h[NS + i4]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f32x4 v0, v1;
      mix4_pair(ma, xv[0][w], xv[1][w], xv[2][w], xv[3][w], fv[w], 0, v0, v1);
#pragma unroll
      for (int i = 0; i < NS; ++i) out[i][w] = pack_fp8x2_lo(v0[i], v1[i]);
      mix4_pair(ma, xv[0][w], xv[1][w], xv[2][w], xv[3][w], fv[w], 2, v0, v1);
#pragma unroll
      for (int i = 0; i < NS; ++i) out[i][w] = pack_fp8x2_hi(out[i][w], v0[i], v1[i]);
    }
    if (v_raw >= cvec) return;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      __builtin_nontemporal_store(out[i], reinterpret_cast<u32x4 *>(yr + ((size_t)i * cvec + v) * 16));
    return;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float f[4], x[NS][4];
    fp8x4_to_f32(fv[w], f);
#pragma unroll
    for (int j = 0; j < NS; ++j) fp8x4_to_f32(xv[j][w], x[j]);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      float a[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a[k] = hpost[i] * f[k];
#pragma unroll
        for (int j = 0; j < NS; ++j) a[k] = fmaf(hres[i][j], x[j][k], a[k]);
      }
      out[i][w] = pack_fp8x4(a[0], a[1], a[2], a[3]);
    }
  }
#pragma unroll
  for (int i = 0; i < NS; ++i)
    __builtin_nontemporal_store(out[i], reinterpret_cast<u32x4 *>(yr + ((size_t)i * cvec + v) * 16));
}

struct Fp8Shape {
  uint32_t cvec, chunks, tasks;
};

bool fp8_shape(int64_t B, int64_t C, Fp8Shape &sh) {
  sh.cvec = (uint32_t)(C / 16);
  sh.chunks = (sh.cvec + 63u) / 64u;
  const uint64_t tasks = (uint64_t)B * sh.chunks;
  if (tasks >= (1ull << 31)) return false;
  sh.tasks = (uint32_t)tasks;
  return true;
}

template <int NS>
hipError_t launch_pre_fp8_n(int64_t B, int64_t C, const void *X, const float *H, void *F,
                            hipStream_t st) {
  Fp8Shape sh;
  if (!fp8_shape(B, C, sh)) return hipErrorInvalidValue;
  pre_fp8_kernel<NS><<<dim3(sh.tasks), 64, 0, st>>>(static_cast<const uint8_t *>(X), H,
                                                    static_cast<uint8_t *>(F), sh.cvec, sh.chunks,
                                                    sh.tasks);
  return hipGetLastError();
}

template <int NS>
hipError_t launch_post_res_fp8_n(int64_t B, int64_t C, const void *X, const void *F,
                                 const float *H, void *Y, hipStream_t st) {
  Fp8Shape sh;
  if (!fp8_shape(B, C, sh)) return hipErrorInvalidValue;
  post_res_fp8_kernel<NS><<<dim3(sh.tasks), 64, 0, st>>>(
      static_cast<const uint8_t *>(X), static_cast<const uint8_t *>(F), H,
      static_cast<uint8_t *>(Y), sh.cvec, sh.chunks, sh.tasks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pre_fp8(int n, int64_t B, int64_t C, const void *X, const float *H,
                          void *F_pre, hipStream_t st) {
  switch (n) {
    case 1: return launch_pre_fp8_n<1>(B, C, X, H, F_pre, st);
    case 2: return launch_pre_fp8_n<2>(B, C, X, H, F_pre, st);
    case 4: return launch_pre_fp8_n<4>(B, C, X, H, F_pre, st);
    case 8: return launch_pre_fp8_n<8>(B, C, X, H, F_pre, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_post_res_fp8(int n, int64_t B, int64_t C, const void *X, const void *F_out,
                               const float *H, void *X_next, hipStream_t st) {
  switch (n) {
    case 1: return launch_post_res_fp8_n<1>(B, C, X, F_out, H, X_next, st);
    case 2: return launch_post_res_fp8_n<2>(B, C, X, F_out, H, X_next, st);
    case 4: return launch_post_res_fp8_n<4>(B, C, X, F_out, H, X_next, st);
    case 8: return launch_post_res_fp8_n<8>(B, C, X, F_out, H, X_next, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhc
