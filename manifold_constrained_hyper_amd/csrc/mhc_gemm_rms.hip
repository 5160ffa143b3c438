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
//    wavefronts of a workgroup share one staged chunk.  The chunk's phi loads
//    are issued before its X loads, so waiting for phi never waits for X.
//  * With PIPE, the X (and phi) loads of chunk i+1 are issued before the
//    MFMAs of chunk i, so each wave keeps requests in flight while it
//    computes (two register buffers).
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
struct GemmTile {
  static constexpr int N = NS * NS + 2 * NS;
  static constexpr int NP = N + 1;
  static constexpr int NB = (N + 15) / 16;
  static constexpr int LDK = KC + 8;                    // padded LDS row (elements)
  static constexpr int T = KC / 32;                     // MFMA k-steps per chunk
  static constexpr int PHI_VEC = (KC * N) / 8;          // 16-byte vectors of phi per chunk
  static constexpr int PV = (PHI_VEC + 255) / 256;      // ... per thread
  static_assert((KC * N) % 8 == 0, "chunk must be whole 16-byte vectors");
};

template <bool NTL>
__device__ __forceinline__ u32x4 ldx(const uint16_t *p) {
  return NTL ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)) : load16(p);
}

// Loads of one K chunk: phi vectors (per thread) and the A operands of the wave.
template <int NS, int MB, int KC, bool NTL, bool XFIRST = false>
struct ChunkRegs {
  using G = GemmTile<NS, MB, KC>;
  u32x4 pw[G::PV];
  bf16x8 xa[MB][G::T];

  __device__ __forceinline__ void load_phi(const uint16_t *phi, int k0, int k_end, int tid) {
    const int valid_vec = (min(KC, k_end - k0) * G::N) / 8;
    const uint16_t *src = phi + (size_t)k0 * G::N;
#pragma unroll
    for (int p = 0; p < G::PV; ++p) {
      const int v = tid + p * 256;
      pw[p] = u32x4{0u, 0u, 0u, 0u};
      if (v < valid_vec) pw[p] = load16(src + (size_t)v * 8);
    }
  }

  __device__ __forceinline__ void load(const uint16_t *phi, const uint16_t *const *xrow, int k0,
                                       int k_end, int tid, int g) {
    if (!XFIRST) load_phi(phi, k0, k_end, tid);
    load_x(xrow, k0, k_end, g);
    if (XFIRST) load_phi(phi, k0, k_end, tid);
  }

  __device__ __forceinline__ void load_x(const uint16_t *const *xrow, int k0, int k_end, int g) {
    if (k0 + KC <= k_end) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < G::T; ++t)
          xa[mb][t] = __builtin_bit_cast(bf16x8, ldx<NTL>(xrow[mb] + k0 + 32 * t + 8 * g));
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < G::T; ++t) {
          const int k = k0 + 32 * t + 8 * g;
          u32x4 w = {0u, 0u, 0u, 0u};
          if (k < k_end) w = ldx<NTL>(xrow[mb] + k);
          xa[mb][t] = __builtin_bit_cast(bf16x8, w);
        }
    }
  }

  // Transposed store of the phi chunk: element (kk, nn) -> phiT[nn][kk].
  __device__ __forceinline__ void stage(uint16_t *phiT, int tid) const {
#pragma unroll
    for (int p = 0; p < G::PV; ++p) {
      const int v = tid + p * 256;
      if (v < G::PHI_VEC) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int e = v * 8 + q;
          const int kk = e / G::N, nn = e - kk * G::N;
          const uint32_t word = pw[p][q >> 1];
          phiT[nn * G::LDK + kk] = (uint16_t)((q & 1) ? (word >> 16) : (word & 0xffffu));
        }
      }
    }
  }
};

template <int NS, int MB, int KC, bool NTL, bool XFIRST>
__device__ __forceinline__ void chunk_mfma(const ChunkRegs<NS, MB, KC, NTL, XFIRST> &c,
                                           const uint16_t *phiT, int m, int g,
                                           f32x4 (&acc)[MB][GemmTile<NS, MB, KC>::NB],
                                           f32x4 (&gram)[MB]) {
  using G = GemmTile<NS, MB, KC>;
#pragma unroll
  for (int t = 0; t < G::T; ++t) {
    bf16x8 b[G::NB];
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
      b[nb] = *reinterpret_cast<const bf16x8 *>(&phiT[(nb * 16 + m) * G::LDK + 32 * t + 8 * g]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.xa[mb][t], b[nb], acc[mb][nb], 0, 0, 0);
      gram[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.xa[mb][t], c.xa[mb][t], gram[mb], 0, 0, 0);
    }
  }
}

template <int NS, int MB, int KC, bool NTL, bool PIPE, bool XFIRST = false>
__global__ __launch_bounds__(256) void gemm_rms_kernel(const uint16_t *__restrict__ X,
                                                       const uint16_t *__restrict__ phi,
                                                       float *__restrict__ ws, int B, int K,
                                                       int kslice) {
  using G = GemmTile<NS, MB, KC>;
  using Regs = ChunkRegs<NS, MB, KC, NTL, XFIRST>;
  __shared__ __attribute__((aligned(16))) uint16_t phiT[G::NB * 16 * G::LDK];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int s = blockIdx.y;
  const int k_begin = s * kslice;
  const int k_end = min(K, k_begin + kslice);
  const int row_base = blockIdx.x * (64 * MB) + wave * (16 * MB);

  // Columns N..NB*16 of the last block are padding; their outputs are never
  // stored, but keep them finite.
  for (int e = tid; e < (G::NB * 16 - G::N) * G::LDK; e += 256) phiT[G::N * G::LDK + e] = 0;

  const uint16_t *xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = min(row_base + mb * 16 + m, B - 1);
    xrow[mb] = X + (size_t)r * K;
  }

  f32x4 acc[MB][G::NB], gram[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    gram[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if constexpr (!PIPE) {
    Regs c;
    for (int k0 = k_begin; k0 < k_end; k0 += KC) {
      c.load(phi, xrow, k0, k_end, tid, g);
      __syncthreads();  // previous chunk's LDS reads are done
      c.stage(phiT, tid);
      __syncthreads();
      chunk_mfma<NS, MB, KC, NTL, XFIRST>(c, phiT, m, g, acc, gram);
    }
  } else {
    Regs c0, c1;
    int k0 = k_begin;
    c0.load(phi, xrow, k0, k_end, tid, g);
    while (k0 < k_end) {
      // chunk in c0; prefetch the next one into c1
      __syncthreads();
      c0.stage(phiT, tid);
      __syncthreads();
      const int k1 = k0 + KC;
      if (k1 < k_end) c1.load(phi, xrow, k1, k_end, tid, g);
      chunk_mfma<NS, MB, KC, NTL, XFIRST>(c0, phiT, m, g, acc, gram);
      if (k1 >= k_end) break;
      __syncthreads();
      c1.stage(phiT, tid);
      __syncthreads();
      const int k2 = k1 + KC;
      if (k2 < k_end) c0.load(phi, xrow, k2, k_end, tid, g);
      chunk_mfma<NS, MB, KC, NTL, XFIRST>(c1, phiT, m, g, acc, gram);
      k0 = k2;
    }
  }

  // D layout of the 16x16 MFMA: lane (m, g) holds rows 4g..4g+3 of column m.
  float *wsl = ws + (size_t)s * B * G::NP;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) {
      const int col = nb * 16 + m;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row_base + mb * 16 + 4 * g + v;
        if (row < B && col < G::N) wsl[(size_t)row * G::NP + col] = acc[mb][nb][v];
      }
    }
    // Gram diagonal (m, m) sits in lane (m, g = m/4), element m%4.
    if (g == (m >> 2)) {
      const int row = row_base + mb * 16 + m;
      if (row < B) wsl[(size_t)row * G::NP + G::N] = gram[mb][m & 3];
    }
  }
}

template <int NS, int MB, int KC, bool NTL, bool PIPE, bool XFIRST = false>
hipError_t launch_typed(const GemmPlan &p, int64_t B, int64_t C, const void *X, const void *phi,
                        float *ws, hipStream_t st) {
  const dim3 grid((uint32_t)p.row_tiles, (uint32_t)p.split);
  gemm_rms_kernel<NS, MB, KC, NTL, PIPE, XFIRST><<<grid, 256, 0, st>>>(
      static_cast<const uint16_t *>(X), static_cast<const uint16_t *>(phi), ws, (int)B,
      (int)(NS * C), (int)p.kslice);
  return hipGetLastError();
}

// Register-path settings (algo 0), chosen by measurement on MI355X at n=4,
// C=7168, B=16384: 128-k chunks, software-pipelined loads, plain
// (cache-allocating) loads of X, about two workgroups per CU.
constexpr int kGemmKC = 128;
constexpr int64_t kGemmTargetWGs = 512;

template <int NS>
hipError_t launch_n(const GemmPlan &p, int64_t B, int64_t C, const void *X, const void *phi,
                    float *ws, hipStream_t st) {
  if (p.algo == 1 && p.phi_parts == 2) {
    if constexpr (NS == 8) return launch_gemm_lds_typed<NS, 1, 128, 2, 2, 2>(p, B, C, X, phi, ws, st);
    else return launch_gemm_lds_typed<NS, 1, 128, 4, 2, 2>(p, B, C, X, phi, ws, st);
  }
  if (p.algo == 1 && p.xreg > 0) {
    if constexpr (NS == 8 || NS == 4) {
      return launch_gemm_xreg_typed<NS, 8, 256, 2>(p, B, C, X, phi, ws, st);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (p.algo == 1 && p.xb == 1 && p.waves == 8) {
    if constexpr (NS == 8) return launch_gemm_lds_typed<NS, 1, 256, 2, 1, 1, 8>(p, B, C, X, phi, ws, st);
    else return launch_gemm_lds_typed<NS, 1, 256, 3, 1, 1, 8>(p, B, C, X, phi, ws, st);
  }
  if (p.algo == 1 && p.waves == 8) {
    if constexpr (NS == 8) return launch_gemm_lds_typed<NS, 1, 128, 3, 2, 1, 8>(p, B, C, X, phi, ws, st);
    else if (p.kc == 256) return launch_gemm_lds_typed<NS, 1, 256, 2, 2, 1, 8>(p, B, C, X, phi, ws, st);
    else return launch_gemm_lds_typed<NS, 1, 128, 4, 2, 1, 8>(p, B, C, X, phi, ws, st);
  }
  if (p.algo == 1 && p.xb == 1) {
    if constexpr (NS == 8) {
      if (p.mb == 2) return launch_gemm_lds_typed<NS, 2, 256, 2, 1, 1>(p, B, C, X, phi, ws, st);
      return launch_gemm_lds_typed<NS, 1, 256, 2, 1, 1>(p, B, C, X, phi, ws, st);
    } else if (p.mb == 2) return launch_gemm_lds_typed<NS, 2, 256, 3, 1, 1>(p, B, C, X, phi, ws, st);
    else return launch_gemm_lds_typed<NS, 1, 256, 4, 1, 1>(p, B, C, X, phi, ws, st);
  }
  if (p.algo == 1) {
    if constexpr (NS == 8) {
      if (p.mb == 2) return launch_gemm_lds_typed<NS, 2, 128, 3, 2, 1>(p, B, C, X, phi, ws, st);
      if (p.kc == 256) return launch_gemm_lds_typed<NS, 1, 256, 2, 2, 1>(p, B, C, X, phi, ws, st);
      return launch_gemm_lds_typed<NS, 1, 128, 4, 2, 1>(p, B, C, X, phi, ws, st);
    } else {
      if (p.kc == 128 && p.stages == 5) return launch_gemm_lds_typed<NS, 1, 128, 5, 2, 1>(p, B, C, X, phi, ws, st);
      if (p.kc == 128 && p.stages == 6) return launch_gemm_lds_typed<NS, 1, 128, 6, 2, 1>(p, B, C, X, phi, ws, st);
      return launch_gemm_lds_typed<NS, 1, 256, 3, 2, 1>(p, B, C, X, phi, ws, st);
    }
  }
  if (p.mb == 2) return launch_typed<NS, 2, kGemmKC, false, true>(p, B, C, X, phi, ws, st);
  return launch_typed<NS, 1, kGemmKC, false, true>(p, B, C, X, phi, ws, st);
}

}  // namespace

GemmPlan plan_gemm_custom(int64_t B, int n, int64_t C, int algo, int mb, int kc, int stages,
                          int64_t target_wgs, int waves) {
  GemmPlan p;
  p.waves = algo == 1 ? waves : 4;
  p.xreg = 0;
  const int64_t K = (int64_t)n * C;
  const int64_t N = (int64_t)n * n + 2 * n;
  const int64_t NB = (N + 15) / 16;
  p.algo = algo;
  p.xb = 2;
  p.phi_parts = 1;
  p.kc = kc;
  p.mb = mb;
  p.stages = stages;
  const int64_t rows = 16 * (int64_t)p.mb * p.waves;
  p.row_tiles = (B + rows - 1) / rows;
  const int64_t kchunks = (K + p.kc - 1) / p.kc;
  int64_t want = (target_wgs + p.row_tiles - 1) / p.row_tiles;
  if (tune(kTuneSplitK) > 0) want = tune(kTuneSplitK);  // tuning override
  if (want < 1) want = 1;
  if (want > kchunks) want = kchunks;
  const int64_t chunks_per_slice = (kchunks + want - 1) / want;
  p.kslice = chunks_per_slice * p.kc;
  p.split = (int)((K + p.kslice - 1) / p.kslice);
  p.partial_bytes = (size_t)p.split * (size_t)B * (size_t)(N + 1) * sizeof(float);
  if (algo == 1) {
    p.phip_offset = (p.partial_bytes + 1023) & ~(size_t)1023;
    p.phip_bytes = (size_t)(kchunks * p.kc / 32) * (size_t)NB * 1024;
    p.zero_offset = p.phip_offset + p.phip_bytes;
    p.total_bytes = p.zero_offset + 256;
  } else {
    p.phip_offset = p.phip_bytes = p.zero_offset = 0;
    p.total_bytes = p.partial_bytes;
  }
  return p;
}

GemmPlan plan_gemm(int64_t B, int n, int64_t C, bool fp8_x, bool phi32) {
  // fp32 phi (bf16 X): X staged through LDS in 128-k chunks, so that the
  // doubled (hi + lo) phi blocks fit the ring: four stages, two at n = 8.
  if (phi32) {
    const int64_t target = tune(kTuneGemmWgs) > 0 ? tune(kTuneGemmWgs) : 256;
    GemmPlan p = plan_gemm_custom(B, n, C, 1, 1, 128, n == 8 ? 2 : 4, target);
    p.phi_parts = 2;
    p.phip_bytes *= 2;
    p.zero_offset = p.phip_offset + p.phip_bytes;
    p.total_bytes = p.zero_offset + 256;
    return p;
  }
  // X staged through LDS (algo 1), one workgroup per CU at a time (the LDS
  // ring is 144-160 KiB); enough workgroups to fill the 256 CUs, and no more
  // K-slices than that needs, since every slice adds (N+1)*4 bytes of
  // partials per row.  E4M3 X: 256-k chunks (16 pieces of 16 bytes per row),
  // 128-row tiles, three stages (two at n = 8, whose phi blocks are larger).
  const int64_t tw = tune(kTuneGemmWaves);
  if (fp8_x) {
    // E4M3 X: eight waves per workgroup by default (measured at n = 8, C = 4096,
    // B = 8192: 85 us against 90 us with four waves of two 16-row blocks and
    // 107-129 us with four waves of one; at n = 4, C = 7168, B = 16384:
    // 96 against 97-100 us).
    const int waves = tw == 4 ? 4 : 8;
    const int64_t target = tune(kTuneGemmWgs) > 0 ? tune(kTuneGemmWgs) : 256;
    int mb = n == 8 ? 1 : 2;  // 128-row tiles: phi per X byte as for bf16 with 64 rows
    const int64_t v = tune(kTuneGemmMb);
    if (v == 1 || v == 2) mb = (int)v;
    int stages = n == 8 ? 2 : (mb == 2 ? 3 : 4);
    if (waves == 8) {  // 8 waves x 16 rows: 128-row tiles
      mb = 1;
      stages = n == 8 ? 2 : 3;
    }
    GemmPlan p = plan_gemm_custom(B, n, C, 1, mb, 256, stages, target, waves);
    p.xb = 1;
    return p;
  }
  // bf16 X: four waves by default (eight measured no faster: 145 against
  // 140-150 us at n = 8, C = 4096, B = 8192; 172 against 169 us at n = 4).
  const int waves = tw == 8 ? 8 : 4;
  int kc = (n == 8) ? 128 : 256;
  int stages = (n == 8) ? 4 : 3;
  if (n != 8 && tune(kTuneGemmKc) == 128 && (tune(kTuneGemmStages) == 5 || tune(kTuneGemmStages) == 6)) {
    kc = 128;  // tuning: 128-k chunks in a 5- or 6-deep ring
    stages = (int)tune(kTuneGemmStages);
  }
  if (tune(kTuneGemmAlgo) == 0)  // tuning override: the register path (1: the LDS path, the default here)
    return plan_gemm_custom(B, n, C, 0, (B >= 1024) ? 2 : 1, kGemmKC, 1, kGemmTargetWGs);
  const int64_t target = tune(kTuneGemmWgs) > 0 ? tune(kTuneGemmWgs) : 256;
  int mb = 1;
  if (waves == 8) {  // 8 waves x 16 rows: 128-row tiles
    if (n == 8) {
      kc = 128;
      stages = 3;
    } else if (tune(kTuneGemmKc) == 256) {
      kc = 256;
      stages = 2;
    } else {
      kc = 128;
      stages = 4;
    }
  } else if (n == 8 && tune(kTuneGemmMb) == 2) {
    mb = 2;  // 128-row tiles at n = 8: half the phi operand traffic per X byte, three stages
    stages = 3;
  } else if (n == 8 && tune(kTuneGemmKc) == 256) {
    kc = 256;  // 512-byte row pieces at n = 8, two stages
    stages = 2;
  }
  if (tune(kTuneGemmXreg) == 2 && (n == 8 || n == 4)) {
    // X and phi through two register sets: eight waves, 256-k chunks, 128-row tiles
    GemmPlan p = plan_gemm_custom(B, n, C, 1, 1, 256, 1, target, 8);
    p.xreg = 2;
    return p;
  }
  return plan_gemm_custom(B, n, C, 1, mb, kc, stages, target, waves);
}

size_t gemm_workspace_bytes(const GemmPlan &p, int64_t B, int n) {
  (void)B;
  (void)n;
  return p.total_bytes;
}

hipError_t launch_gemm_rms(const GemmPlan &p, int n, int64_t B, int64_t C, const void *X,
                           const void *phi, float *ws, hipStream_t st) {
  switch (n) {
    case 1: return launch_n<1>(p, B, C, X, phi, ws, st);
    case 2: return launch_n<2>(p, B, C, X, phi, ws, st);
    case 4: return launch_n<4>(p, B, C, X, phi, ws, st);
    case 8: return launch_n<8>(p, B, C, X, phi, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhc
