// Streaming kernels of the mHC forward: the n -> 1 pre-mix and the fused
// post/res apply.  Both are HBM-bandwidth bound (about 1 flop per byte), so
// the design is about the memory pipeline only:
//
//  * one wavefront owns one (row, chunk) task; a chunk is 64*VPL consecutive
//    16-byte vectors (8 bf16 channels each) of the hidden dimension, so every
//    load/store instruction of a wave touches 1 KiB of contiguous memory per
//    stream;
//  * the row is wave-uniform, so the row's coefficients (n + n*n fp32) are
//    read once per wave with scalar loads and live in SGPRs;
//  * all loads of a task are issued before any arithmetic, keeping
//    (n+1) * VPL 16-byte requests per lane in flight;
//  * inputs are read once, with the non-temporal hint; outputs are written
//    once (the launchers below pick the store hint per kernel).
//
// Math ([mHC-cutile] = page "mHC 算法分析 & cutile 高效实现", section 2.5 and
// the fused apply of section 3.4): fp32 accumulation of bf16 inputs, one
// round-to-nearest-even to bf16 at the end.
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

template <bool NT>
__device__ __forceinline__ u32x4 ld(const void *p) {
  return NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)) : load16(p);
}
template <bool NT>
__device__ __forceinline__ void st(void *p, u32x4 v) {
  if (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
  else
    *reinterpret_cast<u32x4 *>(p) = v;
}

// F_pre[row, c] = sum_i H_pre[row, i] * X[row, i*C + c]
template <int NS, int VPL, int WPB, bool NTL, bool NTS>
__global__ __launch_bounds__(64 * WPB) void pre_kernel(const uint16_t *__restrict__ X,
                                                  const float *__restrict__ H,
                                                  uint16_t *__restrict__ F, uint32_t cvec,
                                                  uint32_t chunks_per_row, uint32_t tasks) {
  constexpr int N = NS * NS + 2 * NS;
  const uint32_t task = (uint32_t)uniform((int)(blockIdx.x * WPB + (threadIdx.x >> 6)));
  if (task >= tasks) return;
  const uint32_t row = task / chunks_per_row;
  const uint32_t chunk = task - row * chunks_per_row;
  const float *h = H + (size_t)row * N;
  float hpre[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) hpre[i] = h[i];

  const char *xr = reinterpret_cast<const char *>(X) + (size_t)row * NS * cvec * 16;
  char *fr = reinterpret_cast<char *>(F) + (size_t)row * cvec * 16;
  const uint32_t v0 = chunk * (64u * VPL) + (threadIdx.x & 63u);

  u32x4 xv[VPL][NS];
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const uint32_t v = v0 + 64u * u;
    if (v < cvec) {
#pragma unroll
      for (int j = 0; j < NS; ++j) xv[u][j] = ld<NTL>(xr + ((size_t)j * cvec + v) * 16);
    }
  }
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const uint32_t v = v0 + 64u * u;
    if (v < cvec) {
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          a0 = fmaf(hpre[j], bf16_lo(xv[u][j][w]), a0);
          a1 = fmaf(hpre[j], bf16_hi(xv[u][j][w]), a1);
        }
        out[w] = pack_bf16x2(a0, a1);
      }
      st<NTS>(fr + (size_t)v * 16, out);
    }
  }
}

// X_next[row, i*C + c] = sum_j H_res[row, i, j] * X[row, j*C + c] + H_post[row, i] * F_out[row, c]
template <int NS, int VPL, int WPB, bool NTL, bool NTS>
__global__ __launch_bounds__(64 * WPB) void post_res_kernel(const uint16_t *__restrict__ X,
                                                       const uint16_t *__restrict__ F,
                                                       const float *__restrict__ H,
                                                       uint16_t *__restrict__ Y, uint32_t cvec,
                                                       uint32_t chunks_per_row, uint32_t tasks) {
  constexpr int N = NS * NS + 2 * NS;
  const uint32_t task = (uint32_t)uniform((int)(blockIdx.x * WPB + (threadIdx.x >> 6)));
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

  const size_t xrow_bytes = (size_t)NS * cvec * 16;
  const char *xr = reinterpret_cast<const char *>(X) + (size_t)row * xrow_bytes;
  const char *fr = reinterpret_cast<const char *>(F) + (size_t)row * cvec * 16;
  char *yr = reinterpret_cast<char *>(Y) + (size_t)row * xrow_bytes;
  const uint32_t v0 = chunk * (64u * VPL) + (threadIdx.x & 63u);

  u32x4 xv[VPL][NS], fv[VPL];
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const uint32_t v = v0 + 64u * u;
    if (v < cvec) {
#pragma unroll
      for (int j = 0; j < NS; ++j) xv[u][j] = ld<NTL>(xr + ((size_t)j * cvec + v) * 16);
      fv[u] = ld<NTL>(fr + (size_t)v * 16);
    }
  }
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const uint32_t v = v0 + 64u * u;
    if (v < cvec) {
      u32x4 out[NS];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f0 = bf16_lo(fv[u][w]), f1 = bf16_hi(fv[u][w]);
        float x0[NS], x1[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          x0[j] = bf16_lo(xv[u][j][w]);
          x1[j] = bf16_hi(xv[u][j][w]);
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          float a0 = hpost[i] * f0, a1 = hpost[i] * f1;
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            a0 = fmaf(hres[i][j], x0[j], a0);
            a1 = fmaf(hres[i][j], x1[j], a1);
          }
          out[i][w] = pack_bf16x2(a0, a1);
        }
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) st<NTS>(yr + ((size_t)i * cvec + v) * 16, out[i]);
    }
  }
}

// Launch shape shared by both kernels: one wave per (row, chunk) task.
struct StreamShape {
  uint32_t cvec, chunks, tasks;
  dim3 grid;
};

template <int VPL, int WPB>
bool stream_shape(int64_t B, int64_t C, StreamShape &sh) {
  sh.cvec = (uint32_t)(C / 8);
  sh.chunks = (sh.cvec + 64u * VPL - 1) / (64u * VPL);
  const uint64_t tasks = (uint64_t)B * sh.chunks;
  if (tasks >= (1ull << 31)) return false;
  sh.tasks = (uint32_t)tasks;
  sh.grid = dim3((uint32_t)((tasks + WPB - 1) / WPB));
  return true;
}

template <int NS, int VPL, int WPB, bool NTL, bool NTS>
hipError_t launch_pre_t(int64_t B, int64_t C, const void *X, const float *H, void *F,
                        hipStream_t st) {
  StreamShape sh;
  if (!stream_shape<VPL, WPB>(B, C, sh)) return hipErrorInvalidValue;
  pre_kernel<NS, VPL, WPB, NTL, NTS><<<sh.grid, 64 * WPB, 0, st>>>(
      static_cast<const uint16_t *>(X), H, static_cast<uint16_t *>(F), sh.cvec, sh.chunks, sh.tasks);
  return hipGetLastError();
}

template <int NS, int VPL, int WPB, bool NTL, bool NTS>
hipError_t launch_post_res_t(int64_t B, int64_t C, const void *X, const void *F, const float *H,
                             void *Y, hipStream_t st) {
  StreamShape sh;
  if (!stream_shape<VPL, WPB>(B, C, sh)) return hipErrorInvalidValue;
  post_res_kernel<NS, VPL, WPB, NTL, NTS><<<sh.grid, 64 * WPB, 0, st>>>(
      static_cast<const uint16_t *>(X), static_cast<const uint16_t *>(F), H,
      static_cast<uint16_t *>(Y), sh.cvec, sh.chunks, sh.tasks);
  return hipGetLastError();
}

// Launch shapes chosen by measurement on MI355X at n=4, C=7168, B=16384 (the
// variants differ only in speed): one 16-byte vector per lane and one wave
// per workgroup; X and F_out read with the non-temporal hint (touched once);
// X_next stored non-temporally, F_pre with plain stores.
template <int NS>
hipError_t launch_pre_n(int64_t B, int64_t C, const void *X, const float *H, void *F,
                        hipStream_t st) {
  return launch_pre_t<NS, 1, 1, true, false>(B, C, X, H, F, st);
}

template <int NS>
hipError_t launch_post_res_n(int64_t B, int64_t C, const void *X, const void *F, const float *H,
                             void *Y, hipStream_t st) {
  return launch_post_res_t<NS, 1, 1, true, true>(B, C, X, F, H, Y, st);
}

}  // namespace

hipError_t launch_pre(int n, int64_t B, int64_t C, const void *X, const float *H, void *F_pre,
                      hipStream_t st) {
  switch (n) {
    case 1: return launch_pre_n<1>(B, C, X, H, F_pre, st);
    case 2: return launch_pre_n<2>(B, C, X, H, F_pre, st);
    case 4: return launch_pre_n<4>(B, C, X, H, F_pre, st);
    case 8: return launch_pre_n<8>(B, C, X, H, F_pre, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_post_res(int n, int64_t B, int64_t C, const void *X, const void *F_out,
                           const float *H, void *X_next, hipStream_t st) {
  switch (n) {
    case 1: return launch_post_res_n<1>(B, C, X, F_out, H, X_next, st);
    case 2: return launch_post_res_n<2>(B, C, X, F_out, H, X_next, st);
    case 4: return launch_post_res_n<4>(B, C, X, F_out, H, X_next, st);
    case 8: return launch_post_res_n<8>(B, C, X, F_out, H, X_next, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhc
