// Fused coefficient product and sum of squares, split over K.
//
// [mHC-cutile] (page "mHC 算法分析 & cutile 高效实现") section 2.1: all
// N = n*n + 2n logits of a row come from one product X_t . phi; section 2.2:
// r needs sum(X_t^2) of the same row; section 3.1 fuses both into one pass
// over X_t; section 5.1 splits K across workgroups because N is tiny and K
// large.  Each workgroup here produces, for its 64*MB rows and its K-slice,
// the partial logits and the partial sum of squares, written to the workspace
// as fp32 [S, B, N+1] (column N = sum of squares).  A second kernel combines
// the S slices in a fixed order.
//
// gfx950 mapping:
//  * v_mfma_f32_16x16x32_bf16 computes a 16-row x 16-column block of logits
//    per 32 k; N = 24 is covered by two column blocks, N = 80 by five.
//  * X feeds the MFMA A operand straight from global memory: lane (m, g)
//    loads 16 bytes = 8 consecutive k of row m.  Each X byte is loaded once.
//  * phi does not fit in LDS (1.4 MB at n=4, C=7168), so it is staged per K
//    chunk, transposed to n-major / k-contiguous, so a lane's B operand
//    (8 consecutive k of one column) is a single 16-byte LDS read.  All four
//    wavefronts of a workgroup share one staged chunk.
//  * The sum of squares rides on the matrix core too: the product of the A
//    operand with itself (the same registers as the B operand) is the 16 x 16
//    Gram block of the rows, whose diagonal is sum_k x^2 accumulated in fp32.
//  * Rows past B are clamped to B-1 for loading (never stored); k past the
//    slice end load as zeros, so ragged B and K need no other special case.
#include "mhc_device.h"
#include "mhc_launch.h"

#include <stdlib.h>

namespace mhc {

namespace {

template <int NS, int MB, int KC>
__global__ __launch_bounds__(256) void gemm_rms_kernel(const uint16_t *__restrict__ X,
                                                       const uint16_t *__restrict__ phi,
                                                       float *__restrict__ ws, int B, int K,
                                                       int kslice) {
  constexpr int N = NS * NS + 2 * NS;
  constexpr int NP = N + 1;
  constexpr int NB = (N + 15) / 16;
  constexpr int LDK = KC + 8;  // padded LDS row, in elements (keeps 16-byte alignment)
  constexpr int T = KC / 32;   // MFMA k-steps per chunk
  static_assert((KC * N) % 8 == 0, "chunk must be whole 16-byte vectors");
  __shared__ __attribute__((aligned(16))) uint16_t phiT[NB * 16 * LDK];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int s = blockIdx.y;
  const int k_begin = s * kslice;
  const int k_end = min(K, k_begin + kslice);
  const int row_base = blockIdx.x * (64 * MB) + wave * (16 * MB);

  // Columns N..NB*16 of the last block are padding; their outputs are never
  // stored, but keep them finite.
  for (int e = tid; e < (NB * 16 - N) * LDK; e += 256) phiT[N * LDK + e] = 0;

  const uint16_t *xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = min(row_base + mb * 16 + m, B - 1);
    xrow[mb] = X + (size_t)r * K;
  }

  f32x4 acc[MB][NB], gram[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    gram[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int k0 = k_begin; k0 < k_end; k0 += KC) {
    // A operands of the whole chunk first, so the HBM requests are in flight
    // while the workgroup stages phi.
    bf16x8 xa[MB][T];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int k = k0 + 32 * t + 8 * g;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (k < k_end) w = load16(xrow[mb] + k);
        xa[mb][t] = __builtin_bit_cast(bf16x8, w);
      }
    }

    __syncthreads();  // previous chunk's LDS reads are done
    {
      const int valid_vec = (min(KC, k_end - k0) * N) / 8;
      const uint16_t *src = phi + (size_t)k0 * N;
      for (int v = tid; v < (KC * N) / 8; v += 256) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (v < valid_vec) w = load16(src + (size_t)v * 8);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int e = v * 8 + q;
          const int kk = e / N, nn = e - kk * N;
          const uint32_t word = w[q >> 1];
          phiT[nn * LDK + kk] = (uint16_t)((q & 1) ? (word >> 16) : (word & 0xffffu));
        }
      }
    }
    __syncthreads();

#pragma unroll
    for (int t = 0; t < T; ++t) {
      bf16x8 b[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        b[nb] = *reinterpret_cast<const bf16x8 *>(&phiT[(nb * 16 + m) * LDK + 32 * t + 8 * g]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb][t], b[nb], acc[mb][nb], 0, 0, 0);
        gram[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[mb][t], xa[mb][t], gram[mb], 0, 0, 0);
      }
    }
  }

  // D layout of the 16x16 MFMA: lane (m, g) holds rows 4g..4g+3 of column m.
  float *wsl = ws + (size_t)s * B * NP;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = nb * 16 + m;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row_base + mb * 16 + 4 * g + v;
        if (row < B && col < N) wsl[(size_t)row * NP + col] = acc[mb][nb][v];
      }
    }
    // Gram diagonal (m, m) sits in lane (m, g = m/4), element m%4.
    if (g == (m >> 2)) {
      const int row = row_base + mb * 16 + m;
      if (row < B) wsl[(size_t)row * NP + N] = gram[mb][m & 3];
    }
  }
}

template <int NS, int MB>
void launch_typed(const GemmPlan &p, int64_t B, int64_t C, const void *X, const void *phi,
                  float *ws, hipStream_t st) {
  constexpr int KC = (NS == 8) ? 128 : 256;
  const dim3 grid((uint32_t)p.row_tiles, (uint32_t)p.split);
  gemm_rms_kernel<NS, MB, KC><<<grid, 256, 0, st>>>(
      static_cast<const uint16_t *>(X), static_cast<const uint16_t *>(phi), ws, (int)B,
      (int)(NS * C), (int)p.kslice);
}

template <int NS>
void launch_n(const GemmPlan &p, int64_t B, int64_t C, const void *X, const void *phi, float *ws,
              hipStream_t st) {
  if (p.mb == 2)
    launch_typed<NS, 2>(p, B, C, X, phi, ws, st);
  else
    launch_typed<NS, 1>(p, B, C, X, phi, ws, st);
}

}  // namespace

GemmPlan plan_gemm(int64_t B, int n, int64_t C) {
  GemmPlan p;
  const int64_t K = (int64_t)n * C;
  p.kc = (n == 8) ? 128 : 256;
  p.mb = (B >= 1024) ? 2 : 1;
  p.row_tiles = (B + 64 * p.mb - 1) / (64 * p.mb);
  const int64_t kchunks = (K + p.kc - 1) / p.kc;
  // Enough workgroups to cover the 256 CUs several times over, but no more
  // K-slices than needed: every slice adds (N+1)*4 bytes of partials per row.
  const int64_t target_wgs = 1024;
  int64_t want = (target_wgs + p.row_tiles - 1) / p.row_tiles;
  if (const char *e = getenv("MHC_SPLIT_K")) {  // tuning override
    const long v = strtol(e, nullptr, 10);
    if (v > 0) want = v;
  }
  if (want < 1) want = 1;
  if (want > kchunks) want = kchunks;
  const int64_t chunks_per_slice = (kchunks + want - 1) / want;
  p.kslice = chunks_per_slice * p.kc;
  p.split = (int)((K + p.kslice - 1) / p.kslice);
  return p;
}

size_t gemm_workspace_bytes(const GemmPlan &p, int64_t B, int n) {
  const int64_t N = (int64_t)n * n + 2 * n;
  return (size_t)p.split * (size_t)B * (size_t)(N + 1) * sizeof(float);
}

hipError_t launch_gemm_rms(const GemmPlan &p, int n, int64_t B, int64_t C, const void *X,
                           const void *phi, float *ws, hipStream_t st) {
  switch (n) {
    case 1: launch_n<1>(p, B, C, X, phi, ws, st); break;
    case 2: launch_n<2>(p, B, C, X, phi, ws, st); break;
    case 4: launch_n<4>(p, B, C, X, phi, ws, st); break;
    case 8: launch_n<8>(p, B, C, X, phi, ws, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mhc
