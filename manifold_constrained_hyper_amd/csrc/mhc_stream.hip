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
//  * outputs are written once with non-temporal stores.
//
// Math ([mHC-cutile] = page "mHC 算法分析 & cutile 高效实现", section 2.5 and
// the fused apply of section 3.4): fp32 accumulation of bf16 inputs, one
// round-to-nearest-even to bf16 at the end.
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

constexpr int kWavesPerBlock = 4;

// F_pre[row, c] = sum_i H_pre[row, i] * X[row, i*C + c]
template <int NS, int VPL>
__global__ __launch_bounds__(256) void pre_kernel(const uint16_t *__restrict__ X,
                                                  const float *__restrict__ H,
                                                  uint16_t *__restrict__ F, uint32_t cvec,
                                                  uint32_t chunks_per_row, uint32_t tasks) {
  constexpr int N = NS * NS + 2 * NS;
  const uint32_t task = (uint32_t)uniform((int)(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)));
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
      for (int j = 0; j < NS; ++j) xv[u][j] = load16(xr + ((size_t)j * cvec + v) * 16);
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
      store16_nt(fr + (size_t)v * 16, out);
    }
  }
}

// X_next[row, i*C + c] = sum_j H_res[row, i, j] * X[row, j*C + c] + H_post[row, i] * F_out[row, c]
template <int NS, int VPL>
__global__ __launch_bounds__(256) void post_res_kernel(const uint16_t *__restrict__ X,
                                                       const uint16_t *__restrict__ F,
                                                       const float *__restrict__ H,
                                                       uint16_t *__restrict__ Y, uint32_t cvec,
                                                       uint32_t chunks_per_row, uint32_t tasks) {
  constexpr int N = NS * NS + 2 * NS;
  const uint32_t task = (uint32_t)uniform((int)(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)));
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
      for (int j = 0; j < NS; ++j) xv[u][j] = load16(xr + ((size_t)j * cvec + v) * 16);
      fv[u] = load16(fr + (size_t)v * 16);
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
      for (int i = 0; i < NS; ++i) store16_nt(yr + ((size_t)i * cvec + v) * 16, out[i]);
    }
  }
}

// Vectors per lane: the candidate that wastes the fewest lanes on the ragged
// end of a row, preferring 2 (two tasks' worth of requests in flight).
int pick_vpl(uint32_t cvec) {
  const int cand[3] = {2, 4, 1};
  int best = 2;
  double best_waste = 2.0;
  for (int c : cand) {
    const uint32_t chunk = 64u * c;
    const uint32_t chunks = (cvec + chunk - 1) / chunk;
    const double waste = double(chunks * chunk - cvec) / double(chunks * chunk);
    if (waste < best_waste - 1e-12) {
      best_waste = waste;
      best = c;
    }
  }
  return best;
}

template <int NS>
hipError_t launch_pre_n(int64_t B, int64_t C, const void *X, const float *H, void *F,
                        hipStream_t st) {
  const uint32_t cvec = (uint32_t)(C / 8);
  const int vpl = pick_vpl(cvec);
  const uint32_t chunks = (cvec + 64u * vpl - 1) / (64u * vpl);
  const uint64_t tasks = (uint64_t)B * chunks;
  if (tasks >= (1ull << 31)) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)((tasks + kWavesPerBlock - 1) / kWavesPerBlock));
  const uint16_t *x = static_cast<const uint16_t *>(X);
  uint16_t *f = static_cast<uint16_t *>(F);
  switch (vpl) {
    case 1: pre_kernel<NS, 1><<<grid, 256, 0, st>>>(x, H, f, cvec, chunks, (uint32_t)tasks); break;
    case 2: pre_kernel<NS, 2><<<grid, 256, 0, st>>>(x, H, f, cvec, chunks, (uint32_t)tasks); break;
    default: pre_kernel<NS, 4><<<grid, 256, 0, st>>>(x, H, f, cvec, chunks, (uint32_t)tasks); break;
  }
  return hipGetLastError();
}

template <int NS>
hipError_t launch_post_res_n(int64_t B, int64_t C, const void *X, const void *F, const float *H,
                             void *Y, hipStream_t st) {
  const uint32_t cvec = (uint32_t)(C / 8);
  const int vpl = pick_vpl(cvec);
  const uint32_t chunks = (cvec + 64u * vpl - 1) / (64u * vpl);
  const uint64_t tasks = (uint64_t)B * chunks;
  if (tasks >= (1ull << 31)) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)((tasks + kWavesPerBlock - 1) / kWavesPerBlock));
  const uint16_t *x = static_cast<const uint16_t *>(X);
  const uint16_t *f = static_cast<const uint16_t *>(F);
  uint16_t *y = static_cast<uint16_t *>(Y);
  switch (vpl) {
    case 1: post_res_kernel<NS, 1><<<grid, 256, 0, st>>>(x, f, H, y, cvec, chunks, (uint32_t)tasks); break;
    case 2: post_res_kernel<NS, 2><<<grid, 256, 0, st>>>(x, f, H, y, cvec, chunks, (uint32_t)tasks); break;
    default: post_res_kernel<NS, 4><<<grid, 256, 0, st>>>(x, f, H, y, cvec, chunks, (uint32_t)tasks); break;
  }
  return hipGetLastError();
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
