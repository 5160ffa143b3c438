// phi packing for the MFMA B operands, and a zero-fill kernel.
//
// The coefficient product of [mHC-cutile] (page "mHC 算法分析 & cutile 高效实现",
// sections 2.1 and 3.1) multiplies X by phi [K, N]; the matrix cores take phi
// as 16-column blocks of 32 k each, one 16-byte operand (8 consecutive k of
// one column) per lane.  pack_phi_kernel rewrites phi once per call into that
// order, so that every kernel that consumes it (the split-K products of
// mhc_gemm_lds.hip, the fused kernel of mhc_post_res_fused.hip) moves its
// operands as contiguous KiB blocks.  The same launch can zero-fill a range
// of the workspace (the fused kernel's hand-off records), which saves a
// launch.
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

// phi [K, N] -> packed B operands: for 32-k step ks and column block nb, lane
// (m, g) of the 1 KiB block holds phi[ks*32 + 8g + j][nb*16 + m], j = 0..7.
// Also clears the 256-byte zero block.
template <int NS>
__global__ __launch_bounds__(256) void pack_phi_kernel(const uint16_t *__restrict__ phi,
                                                       uint16_t *__restrict__ phip,
                                                       uint16_t *__restrict__ zero, int K,
                                                       int ksteps, u32x4 *__restrict__ clr,
                                                       int64_t clr_vecs) {
  // One wave per 32-row k-step.  The step's rows of phi are one contiguous
  // block of 64*N bytes; the wave copies it to LDS with 16-byte loads, then
  // each lane gathers its 8 consecutive k of one column per 16-column block.
  // The grid also zero-fills clr[0, clr_vecs) (16-byte vectors; none when
  // clr_vecs is 0).
  constexpr int N = NS * NS + 2 * NS;
  constexpr int NB = (N + 15) / 16;
  constexpr int PIECES = 4 * N;                // 16-byte pieces per k-step (32 rows x 2N bytes)
  constexpr int PPL = (PIECES + 63) / 64;      // ... per lane
  __shared__ __attribute__((aligned(16))) uint16_t buf[4][32 * N];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && threadIdx.x < 16) store16_plain(zero + threadIdx.x * 8, u32x4{0u, 0u, 0u, 0u});
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < clr_vecs; v += (int64_t)gridDim.x * 256)
    store16_plain(clr + v, u32x4{0u, 0u, 0u, 0u});
  const int ks_raw = blockIdx.x * 4 + wave;
  const int ks = min(ks_raw, ksteps - 1);      // surplus waves redo the last step and store nothing
  const int64_t k0 = (int64_t)ks * 32;
  const int64_t valid_bytes = (min((int64_t)K, k0 + 32) - k0) * (2 * N);  // a multiple of 16 (K % 8 == 0)
  const char *src = reinterpret_cast<const char *>(phi) + k0 * (2 * N);
  char *dst = reinterpret_cast<char *>(buf[wave]);
#pragma unroll
  for (int q = 0; q < PPL; ++q) {
    const int p = lane + 64 * q;
    if (p < PIECES) {
      const u32x4 v = (int64_t)p * 16 < valid_bytes ? load16(reinterpret_cast<const uint16_t *>(src + p * 16))
                                                    : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(dst + p * 16) = v;
    }
  }
  __syncthreads();
  if (ks_raw >= ksteps) return;
  const int kk = 8 * (lane >> 4);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + (lane & 15);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = n < N ? buf[wave][(kk + 2 * q) * N + n] : 0u;
      const uint32_t hi = n < N ? buf[wave][(kk + 2 * q + 1) * N + n] : 0u;
      w[q] = lo | (hi << 16);
    }
    store16_plain(phip + ((int64_t)(ks * NB + nb) * 64 + lane) * 8, u32x4{w[0], w[1], w[2], w[3]});
  }
}

// fp32 phi [K, N] -> packed hi and lo bf16 B operands: for 32-k step ks the
// NB hi blocks (phi_hi = bf16(phi)), then the NB lo blocks (phi_lo =
// bf16(phi - phi_hi)); block layout as in pack_phi_kernel.  Also clears the
// zero block.
template <int NS>
__global__ __launch_bounds__(256) void pack_phi32_kernel(const float *__restrict__ phi,
                                                         uint16_t *__restrict__ phip,
                                                         uint16_t *__restrict__ zero, int K,
                                                         int ksteps) {
  constexpr int N = NS * NS + 2 * NS;
  constexpr int NB = (N + 15) / 16;
  constexpr int PIECES = 8 * N;                // 16-byte pieces per k-step (32 rows x 4N bytes)
  constexpr int PPL = (PIECES + 63) / 64;
  __shared__ __attribute__((aligned(16))) float buf[4][32 * N];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && threadIdx.x < 16) store16_plain(zero + threadIdx.x * 8, u32x4{0u, 0u, 0u, 0u});
  const int ks_raw = blockIdx.x * 4 + wave;
  const int ks = min(ks_raw, ksteps - 1);
  const int64_t k0 = (int64_t)ks * 32;
  const int64_t valid_bytes = (min((int64_t)K, k0 + 32) - k0) * (4 * N);  // a multiple of 16
  const char *src = reinterpret_cast<const char *>(phi) + k0 * (4 * N);
  char *dst = reinterpret_cast<char *>(buf[wave]);
#pragma unroll
  for (int q = 0; q < PPL; ++q) {
    const int p = lane + 64 * q;
    if (p < PIECES) {
      const u32x4 v = (int64_t)p * 16 < valid_bytes ? load16(src + p * 16) : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(dst + p * 16) = v;
    }
  }
  __syncthreads();
  if (ks_raw >= ksteps) return;
  const int kk = 8 * (lane >> 4);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + (lane & 15);
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float f0 = n < N ? buf[wave][(kk + 2 * q) * N + n] : 0.f;
      const float f1 = n < N ? buf[wave][(kk + 2 * q + 1) * N + n] : 0.f;
      wh[q] = pack_bf16x2(f0, f1);
      wl[q] = pack_bf16x2(f0 - bf16_lo(wh[q]), f1 - bf16_hi(wh[q]));  // differences exact in fp32
    }
    store16_plain(phip + ((int64_t)(ks * 2 * NB + nb) * 64 + lane) * 8, u32x4{wh[0], wh[1], wh[2], wh[3]});
    store16_plain(phip + ((int64_t)(ks * 2 * NB + NB + nb) * 64 + lane) * 8, u32x4{wl[0], wl[1], wl[2], wl[3]});
  }
}

}  // namespace

hipError_t launch_pack_phi(int n, int64_t K, int64_t ksteps, const void *phi, void *phip,
                           void *zero, hipStream_t st, void *clear, size_t clear_bytes) {
  const dim3 grid((uint32_t)((ksteps + 3) / 4));  // one wave per 32-row k-step
  const uint16_t *src = static_cast<const uint16_t *>(phi);
  uint16_t *dst = static_cast<uint16_t *>(phip), *z = static_cast<uint16_t *>(zero);
  u32x4 *clr = static_cast<u32x4 *>(clear);
  const int64_t cv = clear ? (int64_t)(clear_bytes / 16) : 0;
  switch (n) {
    case 1: pack_phi_kernel<1><<<grid, 256, 0, st>>>(src, dst, z, (int)K, (int)ksteps, clr, cv); break;
    case 2: pack_phi_kernel<2><<<grid, 256, 0, st>>>(src, dst, z, (int)K, (int)ksteps, clr, cv); break;
    case 4: pack_phi_kernel<4><<<grid, 256, 0, st>>>(src, dst, z, (int)K, (int)ksteps, clr, cv); break;
    case 8: pack_phi_kernel<8><<<grid, 256, 0, st>>>(src, dst, z, (int)K, (int)ksteps, clr, cv); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pack_phi32(int n, int64_t K, int64_t ksteps, const void *phi, void *phip, void *zero,
                             hipStream_t st) {
  const dim3 grid((uint32_t)((ksteps + 3) / 4));  // one wave per 32-row k-step
  const float *src = static_cast<const float *>(phi);
  uint16_t *dst = static_cast<uint16_t *>(phip), *z = static_cast<uint16_t *>(zero);
  switch (n) {
    case 1: pack_phi32_kernel<1><<<grid, 256, 0, st>>>(src, dst, z, (int)K, (int)ksteps); break;
    case 2: pack_phi32_kernel<2><<<grid, 256, 0, st>>>(src, dst, z, (int)K, (int)ksteps); break;
    case 4: pack_phi32_kernel<4><<<grid, 256, 0, st>>>(src, dst, z, (int)K, (int)ksteps); break;
    case 8: pack_phi32_kernel<8><<<grid, 256, 0, st>>>(src, dst, z, (int)K, (int)ksteps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

namespace {
// Streaming stores: with plain ones the one-pass calls that follow ran 8-10 us
// slower per call at n=4, C=7168, B=16384 (401-405 against 392-395 us), the
// cleared lines then sitting dirty in L2 while the pass exchanges its records.
__global__ __launch_bounds__(256) void zero_kernel(u32x4 *__restrict__ p, int64_t nv) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < nv; i += (int64_t)gridDim.x * 256)
    store16_nt(p + i, u32x4{0u, 0u, 0u, 0u});
}
}  // namespace

hipError_t launch_zero(void *p, size_t bytes, hipStream_t st) {
  const int64_t nv = (int64_t)(bytes / 16);
  if (nv <= 0) return hipSuccess;
  const int64_t blocks = (nv + 255) / 256;
  zero_kernel<<<dim3((uint32_t)(blocks < 8192 ? blocks : 8192)), 256, 0, st>>>(static_cast<u32x4 *>(p), nv);
  return hipGetLastError();
}

}  // namespace mhc
