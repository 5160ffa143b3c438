// Post/res apply of one layer fused with the coefficient product of the next.
//
// [mHC-cutile] (page "mHC 算法分析 & cutile 高效实现") section 2.5 produces
// X_{t+1} = H_res X_t + H_post^T F_out; section 2.1 then starts the next
// layer with one product X_{t+1} . phi_{t+1} and section 2.2 with the row
// sums of X_{t+1}^2.  The next layer's product reads exactly what this apply
// writes, so both run in one pass: every X_{t+1} element is multiplied into
// the next layer's logits while it is still on chip, and X_{t+1} is never
// read back for the product.  Per layer this removes one full read of the
// residual stream from HBM.
//
// Work decomposition.  A unit is a 16-row tile times a slice of `spu`
// consecutive 512-channel steps (all n streams of those channels); the S
// slices of a row range cover the hidden size, and unit u is (tile u / S,
// slice u % S).  A persistent grid of G 16-wave workgroups (one per CU)
// takes units round-robin: round j of workgroup g is unit j*G + p(g), where
// p deals each XCD (workgroups are dispatched to the 8 XCDs in turn) a
// contiguous run of units.  At any moment the workgroups are thus working on
// about G consecutive units, i.e. G/S consecutive row tiles: the set of HBM
// pages being streamed stays as compact as in a plain row-major elementwise
// pass.  (With one workgroup per tile sweeping its whole hidden size, 256
// tiles spread over hundreds of MiB are live at once, and the same traffic
// runs about 20 % slower on MI355X.)
//
// Per step (512 channels of one unit), with the loads two steps ahead
// (one step ahead for n = 8, where two register sets do not fit):
//   apply    wave w computes row w of the tile exactly like post_res_kernel
//            (one 16-byte vector = 8 channels per lane and stream, 1 KiB
//            contiguous per load/store instruction), stores X_{t+1} to HBM
//            and drops the same bf16 vectors into an LDS tile
//            [16 rows][n streams][512 channels], 16-byte pieces XOR-swizzled
//            by row so the MFMA operand reads below are conflict-free;
//   product  the step's 16*n MFMA k-steps (32 channels of one stream each)
//            are split over the 16 waves; each reads its A operands (16 rows x
//            8 channels per lane) from LDS and its B operands from the packed
//            copy of phi_{t+1} (see mhc_gemm_lds.hip) and accumulates
//            v_mfma_f32_16x16x32_bf16 plus the Gram block for sum of squares;
//   flush    the 16 waves' accumulators are summed through LDS in wave order
//            (fixed: deterministic) into the unit's partials fp32 [S, B, N+1]
//            of the workspace, which the combine kernel turns into the next
//            layer's logits, r and H.  Every step rewrites its unit's running
//            sum (same thread, same address), so the last write is the unit's
//            total and no memory operation depends on a branch.
// Every wave issues the same memory operations on every step (out-of-range
// lanes and rows use clamped addresses; stores that have no target go to a
// dummy workspace area), which keeps the compiler's memory-counter waits
// exact: the apply of step s waits only for the loads of step s.
//
// The apply arithmetic is that of post_res_kernel (fp32 FMA chain from
// H_post * F_out, one round-to-nearest-even to bf16), so X_{t+1} is bitwise
// what the stand-alone apply writes, and the product consumes those rounded
// values, exactly what a separate product pass would read back.
#include "mhc_device.h"
#include "mhc_launch.h"

#include <atomic>
#include <cstdlib>
#include <type_traits>

namespace mhc {

namespace {

constexpr int kStepCh = 512;          // channels per step: 64 lanes x 8
constexpr int kLdsMax = 160 * 1024;   // LDS of one CU

template <int NS>
struct FusedTile {
  static constexpr int N = NS * NS + 2 * NS;
  static constexpr int NP = N + 1;
  static constexpr int NB = (N + 15) / 16;
  static constexpr int ROW_BYTES = NS * kStepCh * 2;   // one tile row in LDS
  static constexpr int TILE_BYTES = 16 * ROW_BYTES;    // 64 KiB at n=4, 128 KiB at n=8
  static constexpr int KSTEPS = 16 * NS;               // 32-channel MFMA steps per step
  static constexpr int KPW = KSTEPS / 16;              // ... per wave (= NS)
  static constexpr int KB = NS >= 8 ? 2 : (KPW < 4 ? KPW : 4);  // k-steps whose B operands are held at once
  static constexpr int NH = NS + NS * NS;              // H_post and H_res of one row
  static constexpr int HV = (NH + 63) / 64;            // dwords per lane that hold them
  static constexpr int RS = NB * 16 + 1;               // reduction row stride; Gram sum at NB*16
  static constexpr int RED_BYTES = 16 * 16 * RS * 4;   // [16 waves][16 rows][RS] fp32
  // The reduction buffer sits beside the tile when both fit (then the flush
  // of step s-1 overlaps step s); otherwise it reuses the tile buffer.
  static constexpr bool SEPARATE = TILE_BYTES + RED_BYTES <= kLdsMax;
  static constexpr int LDS_BYTES = SEPARATE ? TILE_BYTES + RED_BYTES
                                            : (TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES);
  static constexpr int OPT = (16 * NP + 1023) / 1024;  // flushed sums per thread
  static_assert(LDS_BYTES <= kLdsMax, "LDS budget");
};

struct Step {
  int row0, c0, c_end, slot;
};

// What the kernel reads, writes and multiplies (FusedMode, mhc_launch.h).
template <int MODE>
struct FusedIO {
  static constexpr bool FP8 = MODE == kFusedApplyFp8 || MODE == kFusedCoeffsFp8;
  static constexpr bool APPLY = MODE == kFusedApplyBf16 || MODE == kFusedApplyFp8;
  static constexpr int EB = FP8 ? 1 : 2;  // bytes per element
  using vec = typename std::conditional<FP8, u32x2, u32x4>::type;  // 8 elements per lane
};

template <int NS, int MODE>
__global__ __launch_bounds__(1024) void post_res_next_kernel(
    const uint8_t *__restrict__ X, const uint8_t *__restrict__ F, const float *__restrict__ H,
    uint8_t *__restrict__ Y, const uint16_t *__restrict__ phip, float *__restrict__ ws,
    float *__restrict__ dummy, int B, int C, int spu, int S, int U) {
  using T = FusedTile<NS>;
  using IO = FusedIO<MODE>;
  using vec = typename IO::vec;
  __shared__ __attribute__((aligned(1024))) char lds[T::LDS_BYTES];
  float *red = reinterpret_cast<float *>(lds + (T::SEPARATE ? T::TILE_BYTES : 0));

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int cw = spu * kStepCh;

  // This workgroup's units: p(g) + j*G, j = 0, 1, ...
  const int G = gridDim.x, gi = blockIdx.x;
  const int pg = (gi & 7) * (G >> 3) + min(gi & 7, G & 7) + (gi >> 3);
  if (pg >= U) return;
  const int nsteps = ((U - pg + G - 1) / G) * spu;

  auto step_at = [&](int t) {
    const int j = t / spu, p = t - j * spu;
    const int u = j * G + pg;
    const int tile = u / S, s = u - tile * S;
    const int cb = s * cw;
    return Step{uniform(tile * 16), uniform(cb + p * kStepCh), uniform(min(C, cb + cw)), uniform(s)};
  };

  char *my_lds_row = lds + wave * T::ROW_BYTES;
  const int wslot = (lane ^ (wave & 15)) * 16;  // swizzled 16-byte slot of this lane

  f32x4 acc[T::NB], gram;
  gram = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < T::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads of one step: this wave's row of X_t and F_out and the row's
  // H_post / H_res (lane k holds coefficient k).  Lanes past the slice, and
  // rows past B, read the nearest in-range address instead: they then
  // compute exactly the values the owning lane writes, so their (duplicate)
  // stores rewrite identical bytes, and they enter the LDS tile as zeros.
  auto load_set = [&](vec (&xv)[NS], vec &fv, uint32_t (&hv)[T::HV], const Step &sp) {
    const int rr = uniform(min(sp.row0 + wave, B - 1));
    if constexpr (IO::APPLY) {
      const float *hr = H + (size_t)rr * T::N + NS;
#pragma unroll
      for (int k = 0; k < T::HV; ++k) hv[k] = __builtin_bit_cast(uint32_t, hr[min(k * 64 + lane, T::NH - 1)]);
    }
    const int c = min(sp.c0 + 8 * lane, sp.c_end - 8);
    const uint8_t *xr = X + (size_t)rr * NS * C * IO::EB;
#pragma unroll
    for (int j = 0; j < NS; ++j)
      xv[j] = __builtin_nontemporal_load(reinterpret_cast<const vec *>(xr + ((size_t)j * C + c) * IO::EB));
    if constexpr (IO::APPLY)
      fv = __builtin_nontemporal_load(reinterpret_cast<const vec *>(F + ((size_t)rr * C + c) * IO::EB));
  };

  // Sum the 16 waves' accumulators of step `sp` (in wave order) into its
  // unit's partials.  Threads without a target write the dummy area.
  auto flush = [&](const Step &sp) {
#pragma unroll
    for (int q = 0; q < T::OPT; ++q) {
      const int e = tid + q * 1024;
      const int ec = min(e, 16 * T::NP - 1);
      const int r = ec / T::NP, col = ec - r * T::NP;
      const int rcol = col < T::N ? col : T::NB * 16;
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < 16; ++w) a += red[(w * 16 + r) * T::RS + rcol];
      const int row = sp.row0 + r;
      float *dst = (e < 16 * T::NP && row < B) ? ws + ((size_t)sp.slot * B + row) * T::NP + col
                                               : dummy + e;
      *dst = a;
    }
  };

  auto write_red = [&]() {
    float *rw = red + wave * 16 * T::RS;
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) rw[(4 * g + v) * T::RS + nb * 16 + m] = acc[nb][v];
    if (g == (m >> 2)) rw[m * T::RS + T::NB * 16] = gram[m & 3];
  };

  // One step on the loads in (xv, fv, hv); refills them with step t_pref.
  auto step = [&](int t, vec (&xv)[NS], vec &fv, uint32_t (&hv)[T::HV], int t_pref) {
    const Step sp = step_at(t);
    const int row = sp.row0 + wave;
    const bool live = row < B;
    const int rr = uniform(min(row, B - 1));
    const int c = sp.c0 + 8 * lane;
    const bool in_range = c < sp.c_end;
    const int cst = min(c, sp.c_end - 8);

    // apply (row `rr`, channels c .. c+7 of every stream); the coefficients
    // are broadcast from the lanes of hv.  `out` goes to HBM; the LDS tile
    // gets the same values as bf16 (tile_vec below).
    auto coef = [&](int k) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane((int)hv[k / 64], k % 64));
    };
    vec out[NS];
    if constexpr (MODE == kFusedApplyBf16) {
      if constexpr (NS <= 4) {
        float hpost[NS], hres[NS][NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          hpost[i] = coef(i);
#pragma unroll
          for (int j = 0; j < NS; ++j) hres[i][j] = coef(NS + i * NS + j);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float f0 = bf16_lo(fv[w]), f1 = bf16_hi(fv[w]);
          float x0[NS], x1[NS];
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            x0[j] = bf16_lo(xv[j][w]);
            x1[j] = bf16_hi(xv[j][w]);
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
      } else {
        // n = 8: output stream by output stream, so that only that stream's
        // nine coefficients are held in scalar registers at a time (the same
        // FMA chain per element as above).
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const float hp = coef(i);
          float hr[NS];
#pragma unroll
          for (int j = 0; j < NS; ++j) hr[j] = coef(NS + i * NS + j);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            float a0 = hp * bf16_lo(fv[w]), a1 = hp * bf16_hi(fv[w]);
#pragma unroll
            for (int j = 0; j < NS; ++j) {
              a0 = fmaf(hr[j], bf16_lo(xv[j][w]), a0);
              a1 = fmaf(hr[j], bf16_hi(xv[j][w]), a1);
            }
            out[i][w] = pack_bf16x2(a0, a1);
          }
        }
      }
    } else if constexpr (MODE == kFusedApplyFp8) {
      // E4M3: each 8-byte vector is two words of four channels; the same FMA
      // chain per element as post_res_fp8_kernel, then the E4M3 result is
      // widened (exactly) for the tile.
      if constexpr (NS <= 4) {
        float hpost[NS], hres[NS][NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          hpost[i] = coef(i);
#pragma unroll
          for (int j = 0; j < NS; ++j) hres[i][j] = coef(NS + i * NS + j);
        }
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const f32x2 fl = fp8_lo2(fv[d]), fh = fp8_hi2(fv[d]);
          const float f[4] = {fl[0], fl[1], fh[0], fh[1]};
          float x[NS][4];
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            const f32x2 xl = fp8_lo2(xv[j][d]), xh = fp8_hi2(xv[j][d]);
            x[j][0] = xl[0];
            x[j][1] = xl[1];
            x[j][2] = xh[0];
            x[j][3] = xh[1];
          }
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            float a[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              a[k] = hpost[i] * f[k];
#pragma unroll
              for (int j = 0; j < NS; ++j) a[k] = fmaf(hres[i][j], x[j][k], a[k]);
            }
            out[i][d] = pack_fp8x4(a[0], a[1], a[2], a[3]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const float hp = coef(i);
          float hr[NS];
#pragma unroll
          for (int j = 0; j < NS; ++j) hr[j] = coef(NS + i * NS + j);
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const f32x2 fl = fp8_lo2(fv[d]), fh = fp8_hi2(fv[d]);
            float a[4] = {hp * fl[0], hp * fl[1], hp * fh[0], hp * fh[1]};
#pragma unroll
            for (int j = 0; j < NS; ++j) {
              const f32x2 xl = fp8_lo2(xv[j][d]), xh = fp8_hi2(xv[j][d]);
              a[0] = fmaf(hr[j], xl[0], a[0]);
              a[1] = fmaf(hr[j], xl[1], a[1]);
              a[2] = fmaf(hr[j], xh[0], a[2]);
              a[3] = fmaf(hr[j], xh[1], a[3]);
            }
            out[i][d] = pack_fp8x4(a[0], a[1], a[2], a[3]);
          }
        }
      }
    }
    // Stream i of the LDS tile (bf16): the apply's output, or X itself; the
    // E4M3 values widen exactly.  Taken at the LDS write, before the refill
    // overwrites xv, so no second copy is held across the stores.
    auto tile_vec = [&](int i) -> u32x4 {
      if constexpr (MODE == kFusedApplyBf16) return out[i];
      else if constexpr (MODE == kFusedApplyFp8) return fp8x8_to_bf16(out[i]);
      else if constexpr (MODE == kFusedCoeffsFp8) return fp8x8_to_bf16(xv[i]);
      else return xv[i];
    };
    // B operands of this wave's k-steps (global, L2-resident), in groups of
    // KB k-steps (all of them for n <= 4; for n = 8 the later groups are
    // loaded after the earlier ones are consumed).
    bf16x8 b[T::KB][T::NB];
    auto load_b = [&](int q0) {
#pragma unroll
      for (int q = 0; q < T::KB; ++q) {
        const int ks = wave * T::KPW + q0 + q;       // 0 .. 16*NS-1 within the step
        const int i = ks >> 4, ts = ks & 15;         // stream, 32-channel sub-step
        const int cs = sp.c0 + 32 * ts;
        const int kstep = (i * C + min(cs, C - 32)) >> 5;  // clamped in range; such steps add zero
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
          b[q][nb] = __builtin_bit_cast(bf16x8, load16(phip + ((size_t)(kstep * T::NB + nb) * 64 + lane) * 8));
      }
    };
    if constexpr (IO::APPLY) {
      uint8_t *yr = Y + (size_t)rr * NS * C * IO::EB;
#pragma unroll
      for (int i = 0; i < NS; ++i)
        __builtin_nontemporal_store(out[i], reinterpret_cast<vec *>(yr + ((size_t)i * C + cst) * IO::EB));
    }
    // The first B group is issued before the refill (waiting for it then
    // never waits for the refill), except for n = 8, where holding it across
    // the refill would not fit the register budget.
    if constexpr (NS < 8) load_b(0);

    __syncthreads();  // the previous step's product is done with the tile (and has written red)
    if constexpr (T::SEPARATE) flush(step_at(t > 0 ? t - 1 : 0));
#pragma unroll
    for (int i = 0; i < NS; ++i)
      *reinterpret_cast<u32x4 *>(my_lds_row + i * (kStepCh * 2) + wslot) =
          (in_range && live) ? tile_vec(i) : u32x4{0u, 0u, 0u, 0u};
    load_set(xv, fv, hv, step_at(t_pref));
    if constexpr (NS >= 8) load_b(0);
    __syncthreads();  // the tile is complete (and the flush has read red)

    // A unit's sums start from zero at its first step.
    const bool first = (t % spu) == 0;
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb) acc[nb] = first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[nb];
    gram = first ? f32x4{0.f, 0.f, 0.f, 0.f} : gram;
    // k-steps past the range read zeros from the tile, so they add nothing.
#pragma unroll
    for (int q0 = 0; q0 < T::KPW; q0 += T::KB) {
      if (q0 > 0) load_b(q0);
#pragma unroll
      for (int q = 0; q < T::KB; ++q) {
        const int ks = wave * T::KPW + q0 + q;
        const int i = ks >> 4, ts = ks & 15;
        const int piece = (4 * ts + g) ^ m;
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(lds + m * T::ROW_BYTES + i * (kStepCh * 2) + piece * 16);
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[q][nb], acc[nb], 0, 0, 0);
        gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, gram, 0, 0, 0);
      }
    }
    if constexpr (T::SEPARATE) {
      write_red();  // flushed after the next step's first barrier
    } else {
      __syncthreads();  // every wave is done with the tile, which now holds red
      write_red();
      __syncthreads();
      flush(sp);        // the next step's first barrier orders it before the tile is rewritten
    }
  };

  const int tl = nsteps - 1;
  if constexpr (NS >= 8) {
    // n = 8: one register set (two would not fit 128 VGPRs).
    vec xa[NS], fa;
    uint32_t ha[T::HV];
    load_set(xa, fa, ha, step_at(0));
    for (int t = 0; t < nsteps; ++t) step(t, xa, fa, ha, min(t + 1, tl));
  } else {
    // Two register sets: the loads of step t+2 are issued while step t is
    // applied and multiplied, so each wave has two steps of loads in flight.
    // The loop always runs both steps (an odd last step runs after it), so
    // the waits at the top of each step only cover the set used there.
    vec xa[NS], fa, xb[NS], fb;
    uint32_t ha[T::HV], hb[T::HV];
    load_set(xa, fa, ha, step_at(0));
    load_set(xb, fb, hb, step_at(min(1, tl)));
    int t = 0;
    for (; t + 1 < nsteps; t += 2) {
      step(t, xa, fa, ha, min(t + 2, tl));
      step(t + 1, xb, fb, hb, min(t + 3, tl));
    }
    if (t < nsteps) step(t, xa, fa, ha, tl);
  }
  if constexpr (T::SEPARATE) {
    __syncthreads();
    flush(step_at(tl));
  }
}

// Compute units of the current device (cached per device id).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace

template <int NS, int MODE>
hipError_t launch_post_res_next_typed(int64_t B, int64_t C, int spu, int split, int grid_cap,
                                      const void *X, const void *F, const float *H, void *Y,
                                      const void *phip, float *ws, float *dummy, hipStream_t st) {
  const int64_t U = ((B + 15) / 16) * (int64_t)split;
  const int G = (int)(U < grid_cap ? U : grid_cap);
  post_res_next_kernel<NS, MODE><<<dim3((uint32_t)G), 1024, 0, st>>>(
      static_cast<const uint8_t *>(X), static_cast<const uint8_t *>(F), H,
      static_cast<uint8_t *>(Y), static_cast<const uint16_t *>(phip), ws, dummy, (int)B, (int)C,
      spu, split, (int)U);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int n, int64_t B, int64_t C, int spu, int split, int cap, const void *X,
                       const void *F, const float *H, void *Y, const void *phip, float *ws,
                       float *dummy, hipStream_t st) {
  switch (n) {
    case 1: return launch_post_res_next_typed<1, MODE>(B, C, spu, split, cap, X, F, H, Y, phip, ws, dummy, st);
    case 2: return launch_post_res_next_typed<2, MODE>(B, C, spu, split, cap, X, F, H, Y, phip, ws, dummy, st);
    case 4: return launch_post_res_next_typed<4, MODE>(B, C, spu, split, cap, X, F, H, Y, phip, ws, dummy, st);
    case 8: return launch_post_res_next_typed<8, MODE>(B, C, spu, split, cap, X, F, H, Y, phip, ws, dummy, st);
    default: return hipErrorInvalidValue;
  }
}

FusedPlan plan_post_res_next(int64_t B, int n, int64_t C) {
  FusedPlan p;
  const int64_t N = (int64_t)n * n + 2 * n, NB = (N + 15) / 16, K = (int64_t)n * C;
  p.row_tiles = (B + 15) / 16;
  // Steps per unit: the largest divisor of the row's step count that still
  // leaves at least 7 slices (fewer when the row is shorter), so that the
  // ~256 resident workgroups cover at most ~37 row tiles at a time while the
  // partial sums stay small (7 x B x (N+1) fp32).  MHC_FUSED_SPU overrides
  // (any value >= 1; one that does not divide the step count leaves empty
  // steps at the end of the last slice, which add nothing).
  const int64_t steps = (C + kStepCh - 1) / kStepCh;
  const int64_t want = steps < 7 ? steps : 7;
  int64_t spu = 1;
  for (int64_t d = 1; d <= steps; ++d)
    if (steps % d == 0 && steps / d >= want) spu = d;
  if (const char *e = std::getenv("MHC_FUSED_SPU")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1 && v <= steps) spu = v;
  }
  p.cw = (int)(spu * kStepCh);
  p.split = (int)((steps + spu - 1) / spu);
  p.partial_bytes = (size_t)p.split * (size_t)B * (size_t)(N + 1) * sizeof(float);
  p.ksteps = (K + 31) / 32;
  p.dummy_offset = (p.partial_bytes + 1023) & ~(size_t)1023;
  p.dummy_bytes = (size_t)((16 * (N + 1) + 1023) / 1024) * 1024 * sizeof(float);
  p.phip_offset = p.dummy_offset + p.dummy_bytes;
  p.phip_bytes = (size_t)p.ksteps * (size_t)NB * 1024;
  p.zero_offset = p.phip_offset + p.phip_bytes;
  p.total_bytes = p.zero_offset + 256;
  return p;
}

hipError_t launch_post_res_next(const FusedPlan &p, int n, int mode, int64_t B, int64_t C,
                                const void *X, const void *F, const float *H, void *Y,
                                const void *phi_next, void *ws_base, hipStream_t st) {
  char *base = static_cast<char *>(ws_base);
  void *phip = base + p.phip_offset;
  hipError_t e = launch_pack_phi(n, (int64_t)n * C, p.ksteps, phi_next, phip, base + p.zero_offset, st);
  if (e != hipSuccess) return e;
  float *ws = reinterpret_cast<float *>(base);
  float *dummy = reinterpret_cast<float *>(base + p.dummy_offset);
  const int spu = p.cw / kStepCh;
  int cap = device_cus();
  if (const char *env = std::getenv("MHC_FUSED_WGS")) {
    const long v = std::strtol(env, nullptr, 10);
    if (v >= 1 && v <= 65535) cap = (int)v;
  }
  switch (mode) {
    case kFusedApplyBf16: return launch_mode<kFusedApplyBf16>(n, B, C, spu, p.split, cap, X, F, H, Y, phip, ws, dummy, st);
    case kFusedApplyFp8: return launch_mode<kFusedApplyFp8>(n, B, C, spu, p.split, cap, X, F, H, Y, phip, ws, dummy, st);
    case kFusedCoeffsFp8: return launch_mode<kFusedCoeffsFp8>(n, B, C, spu, p.split, cap, X, F, H, Y, phip, ws, dummy, st);
    case kFusedCoeffsBf16: return launch_mode<kFusedCoeffsBf16>(n, B, C, spu, p.split, cap, X, F, H, Y, phip, ws, dummy, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhc
