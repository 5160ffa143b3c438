// Small-B (decode) path of mhc_coeffs (and mhc_coeffs_fp8): steps (1)-(3) in
// one launch.
//
// [mHC-cutile] (page "mHC 算法分析 & cutile 高效实现") section 2.1: one
// product logits = X_t . phi for all N columns; section 2.2: the row sums of
// X_t^2; sections 2.3-2.4: the per-row finish (mhc_finish.h).  Section 3.2
// notes that at decode sizes these steps are launch-bound; this kernel folds
// the split-K reduction and the finish into the product's launch.
//
// Grid: (16-row tiles) x (K-slices of `kslice` elements), 4 waves each.
//   product  the workgroup stages its slice of phi [kslice, N] in LDS with
//            16-byte loads (the rows of a slice are one contiguous block of
//            phi, so no packed copy is needed), transposed on the way in so
//            that a column's k values are contiguous and each B operand is
//            one 16-byte LDS read; wave w takes k-steps w*KSW .. w*KSW+KSW-1
//            of the slice, with its A operands (16 rows x 8 consecutive k per
//            lane) loaded straight from X_t, all of them issued before the
//            first multiply.  v_mfma_f32_16x16x32_bf16 accumulates the logits
//            and the Gram block whose diagonal is the sum of squares.  The
//            biases are staged in LDS at the start, so the finish waits on
//            no global load.
//   partial  the 4 waves' sums are added through LDS in wave order and the
//            tile's [16, N+1] partial is written to the workspace [S, B, N+1].
//   arrival  each workgroup writes its partial with agent-scope stores (they
//            go through to the device coherence point), waits until they have
//            completed, then writes the call's epoch into its own flag word
//            (one per tile and slice) and waits for that too.  Wave 0 then
//            reads the tile's S flags: a workgroup that finds all of them
//            carrying this call's epoch adds the S partials in slice order
//            0..S-1 (fixed order: the result does not depend on which
//            workgroup does it) and runs the finish for the tile's rows.
//            Since every workgroup's flag is complete before it reads the
//            others', the last one to arrive always sees all flags; if two
//            see them, both write the same bits.  No counter, no atomic
//            read-modify-write, no fence that writes back the L2.
//
// fp32 phi (the *_phi32 calls): the slice is split while it is staged into
// two bf16 arrays, phi_hi = bf16(phi) and phi_lo = bf16(phi - phi_hi), kept
// row-major (each B operand gathered from 8 two-byte LDS reads), and every
// block takes two MFMAs, X.phi_hi + X.phi_lo, into one accumulator.
//
// The epoch is a process-wide 64-bit counter from a start that differs
// between runs, so flags left in a workspace by earlier calls (or any other
// contents) never match the current call: the workspace needs no
// initialisation.  The workgroup that combines a tile clears its flags
// afterwards, so replaying the same launch (same epoch) works as well.
#include "mhc_device.h"
#include "mhc_finish.h"
#include "mhc_launch.h"

#include <atomic>
#include <chrono>
#include <cstdlib>

namespace mhc {

namespace {

template <int NS>
struct SmallTile {
  static constexpr int N = NS * NS + 2 * NS;
  static constexpr int NP = N + 1;
  static constexpr int NB = (N + 15) / 16;
  static constexpr int RS = NB * 16 + 1;            // reduction row stride; Gram sum at NB*16
  static constexpr int KS = kSmallKSlice<NS>();     // K elements per slice (at most)
  static constexpr int KSW = KS / 128;              // k-steps per wave (4 waves x 32 k)
  static constexpr int EPT = (16 * NP + 255) / 256;    // tile sums per thread in the combine
  static_assert(KS % 128 == 0, "slice splits evenly over 4 waves");
  // Transposed bf16 staging: column col's k values at [col * LDK + k].  A unit
  // is G consecutive k of CW columns: 8 columns (G = 4) when N % 8 == 0, one
  // 16-byte piece per k row; otherwise all N columns of G = 8 rows (G*N/8
  // contiguous pieces).
  static constexpr int LDK = KS + 8;
  static constexpr bool CHUNKED = N % 8 == 0;
  static constexpr int G = CHUNKED ? 4 : 8;
  static constexpr int CW = CHUNKED ? 8 : N;
  static constexpr int UP = G * CW / 8;                  // 16-byte pieces per unit
  static constexpr int UNITS = (KS / G) * (N / CW);
  static constexpr int UPT = (UNITS + 255) / 256;        // units per thread
};

template <int NS, bool FP8X, bool P32>
__global__ __launch_bounds__(256) void coeffs_small_kernel(
    const uint8_t *__restrict__ X, const void *__restrict__ phi_v, int B, int K, int S,
    float inv_k, float alpha_pre, float alpha_post, float alpha_res,
    const float *__restrict__ b_pre, const float *__restrict__ b_post,
    const float *__restrict__ b_res, float *__restrict__ logits, float *__restrict__ r_out,
    float *__restrict__ H, float *ws, unsigned long long *flags, unsigned long long epoch) {
  using T = SmallTile<NS>;
  __shared__ __attribute__((aligned(16))) uint16_t phs[P32 ? 2 : 1][P32 ? T::KS * T::N : T::N * T::LDK];
  __shared__ float red[4 * 16 * T::RS];
  __shared__ float sums[16 * T::NP];
  __shared__ float bsh[T::N];  // b_pre, b_post, b_res
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x, s = blockIdx.y;
  const int row0 = tile * 16;
  const int k_lo = s * T::KS;
  const int k_hi = min(K, k_lo + T::KS);
  if (tid < T::N) bsh[tid] = tid < NS ? b_pre[tid] : (tid < 2 * NS ? b_post[tid - NS] : b_res[tid - 2 * NS]);

  // A operands of this wave's k-steps: row row0+m (rows past B read row
  // B-1; their results are not written), k = step*32 + 8g .. +7 (zero past
  // the slice).
  // X in E4M3 (FP8X) is widened exactly to bf16 for the matrix core.
  constexpr int EB = FP8X ? 1 : 2;
  const uint8_t *xr = X + (size_t)min(row0 + m, B - 1) * K * EB;
  bf16x8 a[T::KSW];
#pragma unroll
  for (int q = 0; q < T::KSW; ++q) {
    const int k = k_lo + (wave * T::KSW + q) * 32 + 8 * g;
    u32x4 v;
    if constexpr (FP8X)
      v = fp8x8_to_bf16(*reinterpret_cast<const u32x2 *>(xr + min(k, K - 8)));
    else
      v = load16(xr + (size_t)min(k, K - 8) * 2);
    a[q] = __builtin_bit_cast(bf16x8, k < k_hi ? v : u32x4{0u, 0u, 0u, 0u});
  }

  // phi rows [k_lo, k_hi) into LDS, zero past k_hi.  (k_hi - k_lo) is a
  // multiple of 8, so a unit's G rows lie wholly below k_hi or wholly past
  // it.  All of a thread's loads are issued before the first LDS store.
  if constexpr (!P32) {
    const uint16_t *src = static_cast<const uint16_t *>(phi_v) + (size_t)k_lo * T::N;
    constexpr int CPR = T::N / T::CW;  // column chunks per k row
    u32x4 v[T::UPT][T::UP];
#pragma unroll
    for (int q = 0; q < T::UPT; ++q) {
      const int u = min(tid + 256 * q, T::UNITS - 1);
      const int kg = u / CPR, c0 = (u - kg * CPR) * T::CW;
      const int k0 = k_lo + kg * T::G < k_hi ? kg * T::G : 0;  // units past k_hi read row 0 (zeroed below)
#pragma unroll
      for (int t = 0; t < T::UP; ++t) {
        // CHUNKED: piece t is row k0+t, columns c0..c0+7; otherwise piece t
        // of the G full rows from k0.
        const size_t off = T::CHUNKED ? (size_t)(k0 + t) * T::N + c0 : (size_t)k0 * T::N + 8 * t;
        v[q][t] = load16(src + off);
      }
    }
#pragma unroll
    for (int q = 0; q < T::UPT; ++q) {
      const int u = tid + 256 * q;
      if (u < T::UNITS) {
        const int kg = u / CPR, c0 = (u - kg * CPR) * T::CW;
        const int k0 = kg * T::G;
        const bool valid = k_lo + k0 < k_hi;
#pragma unroll
        for (int j = 0; j < T::CW; ++j) {
          uint32_t w[T::G / 2];
#pragma unroll
          for (int t = 0; t < T::G / 2; ++t) {
            // elements (k0 + 2t, c0 + j) and (k0 + 2t + 1, c0 + j) of the unit
            const int el = T::CHUNKED ? (2 * t) * 8 + j : (2 * t) * T::N + j;
            const int eh = T::CHUNKED ? (2 * t + 1) * 8 + j : (2 * t + 1) * T::N + j;
            const uint32_t lo = (v[q][el >> 3][(el & 7) >> 1] >> (16 * (el & 1))) & 0xffffu;
            const uint32_t hi = (v[q][eh >> 3][(eh & 7) >> 1] >> (16 * (eh & 1))) & 0xffffu;
            w[t] = valid ? (lo | (hi << 16)) : 0u;
          }
          uint16_t *dst = phs[0] + (c0 + j) * T::LDK + k0;
          if constexpr (T::G == 4) {
            *reinterpret_cast<u32x2 *>(dst) = u32x2{w[0], w[1]};
          } else {
            *reinterpret_cast<u32x4 *>(dst) = u32x4{w[0], w[1], w[2], w[3]};
          }
        }
      }
    }
  } else {
    // fp32 phi: 16-byte pieces of 4 values, split into hi and lo halves of 8
    // bytes each; loads issued in batches of 8 pieces per thread.
    constexpr int PIECES32 = T::KS * T::N / 4;
    constexpr int PPT32 = (PIECES32 + 255) / 256;
    constexpr int BATCH = 8;
    const int valid = (k_hi - k_lo) * T::N * 4;
    const char *src = reinterpret_cast<const char *>(static_cast<const float *>(phi_v) + (size_t)k_lo * T::N);
#pragma unroll
    for (int q0 = 0; q0 < PPT32; q0 += BATCH) {
      u32x4 v[BATCH];
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        const int p = tid + 256 * (q0 + q);
        if (q0 + q < PPT32) v[q] = load16(src + (size_t)min(p * 16, valid - 16));
      }
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        const int p = tid + 256 * (q0 + q);
        if (q0 + q < PPT32 && p < PIECES32) {
          const u32x4 w = p * 16 < valid ? v[q] : u32x4{0u, 0u, 0u, 0u};
          const float f0 = __uint_as_float(w[0]), f1 = __uint_as_float(w[1]);
          const float f2 = __uint_as_float(w[2]), f3 = __uint_as_float(w[3]);
          const uint32_t h01 = pack_bf16x2(f0, f1), h23 = pack_bf16x2(f2, f3);
          const uint32_t l01 = pack_bf16x2(f0 - bf16_lo(h01), f1 - bf16_hi(h01));  // exact differences
          const uint32_t l23 = pack_bf16x2(f2 - bf16_lo(h23), f3 - bf16_hi(h23));
          *reinterpret_cast<u32x2 *>(phs[0] + p * 4) = u32x2{h01, h23};
          *reinterpret_cast<u32x2 *>(phs[1] + p * 4) = u32x2{l01, l23};
        }
      }
    }
  }
  __syncthreads();

  f32x4 acc[T::NB], gram = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < T::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < T::KSW; ++q) {
    const int kk = (wave * T::KSW + q) * 32 + 8 * g;  // row of phs
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb) {
      const int col = nb * 16 + m;
      if constexpr (!P32) {
        const u32x4 w = col < T::N ? *reinterpret_cast<const u32x4 *>(phs[0] + col * T::LDK + kk)
                                   : u32x4{0u, 0u, 0u, 0u};
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], __builtin_bit_cast(bf16x8, w), acc[nb], 0, 0, 0);
      } else {
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = col < T::N ? phs[part][(kk + 2 * j) * T::N + col] : 0u;
            const uint32_t hi = col < T::N ? phs[part][(kk + 2 * j + 1) * T::N + col] : 0u;
            w[j] = lo | (hi << 16);
          }
          const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], b, acc[nb], 0, 0, 0);
        }
      }
    }
    gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], a[q], gram, 0, 0, 0);
  }

  // The 4 waves' sums, in wave order, into this slice's partial.
  {
    float *rw = red + wave * 16 * T::RS;
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) rw[(4 * g + v) * T::RS + nb * 16 + m] = acc[nb][v];
    if (g == (m >> 2)) rw[m * T::RS + T::NB * 16] = gram[m & 3];
  }
  __syncthreads();
  const size_t slice = (size_t)B * T::NP;
  const int rows = min(16, B - row0);
  if (S == 1) {
    // One slice: this workgroup holds the tile's whole sums.
    for (int e = tid; e < rows * T::NP; e += 256) {
      const int r = e / T::NP, col = e - r * T::NP;
      const int rcol = col < T::N ? col : T::NB * 16;
      const float v = ((red[(0 * 16 + r) * T::RS + rcol] + red[(1 * 16 + r) * T::RS + rcol]) +
                       red[(2 * 16 + r) * T::RS + rcol]) + red[(3 * 16 + r) * T::RS + rcol];
      sums[e] = v;
      if (col < T::N) logits[(size_t)(row0 + r) * T::N + col] = v;
    }
    __syncthreads();
    const int lr = tid / NS, i = tid % NS;
    if (lr < rows)
      finish_row<NS>(sums + lr * T::NP, row0 + lr, i, inv_k, alpha_pre, alpha_post, alpha_res,
                     bsh, bsh + NS, bsh + 2 * NS, r_out, H);
    return;
  }
  for (int e = tid; e < 16 * T::NP; e += 256) {
    const int r = e / T::NP, col = e - r * T::NP;
    const int rcol = col < T::N ? col : T::NB * 16;
    const float v = ((red[(0 * 16 + r) * T::RS + rcol] + red[(1 * 16 + r) * T::RS + rcol]) +
                     red[(2 * 16 + r) * T::RS + rcol]) + red[(3 * 16 + r) * T::RS + rcol];
    if (row0 + r < B)
      __hip_atomic_store(ws + (size_t)s * slice + (size_t)(row0 + r) * T::NP + col, v,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Arrival: this workgroup's partial is complete, then its flag is.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  unsigned long long *tflags = flags + (size_t)tile * S;
  if (wave == 0) {
    if (lane == 0) __hip_atomic_store(tflags + s, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const unsigned long long f =
        __hip_atomic_load(tflags + min(lane, S - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool arrived = lane >= S || f == epoch;
    const unsigned long long missing = __builtin_amdgcn_ballot_w64(!arrived);  // whole wave votes
    if (lane == 0) is_last = missing == 0;
  }
  __syncthreads();
  if (!is_last) return;

  // Last slice of the tile: add the S partials in slice order.  A thread's
  // loads for kCombineBatch slices of all its elements are issued before any
  // is added (one memory round trip up to 32 slices at n <= 4).
  const float *base = ws + (size_t)row0 * T::NP;
  const int nel = rows * T::NP;
  constexpr int kCombineBatch = combine_batch(T::EPT);
  float tot[T::EPT];
#pragma unroll
  for (int q = 0; q < T::EPT; ++q) tot[q] = 0.f;
  for (int s0 = 0; s0 < S; s0 += kCombineBatch) {
    float v[kCombineBatch][T::EPT];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j)
#pragma unroll
      for (int q = 0; q < T::EPT; ++q)
        v[j][q] = __hip_atomic_load(base + (size_t)min(s0 + j, S - 1) * slice + min(tid + 256 * q, nel - 1),
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j)
#pragma unroll
      for (int q = 0; q < T::EPT; ++q)
        if (s0 + j < S) tot[q] += v[j][q];
  }
#pragma unroll
  for (int q = 0; q < T::EPT; ++q) {
    const int e = tid + 256 * q;
    if (e < nel) {
      sums[e] = tot[q];
      const int r = e / T::NP, col = e - r * T::NP;
      if (col < T::N) logits[(size_t)(row0 + r) * T::N + col] = tot[q];
    }
  }
  // Every slice of this call has arrived, so no workgroup reads the tile's
  // flags any more: clear them, so that a replay of the same launch (same
  // epoch, e.g. from a captured graph) starts from cleared flags.
  if (wave == 0 && lane < S)
    __hip_atomic_store(tflags + lane, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int lr = tid / NS, i = tid % NS;
  if (lr < rows)
    finish_row<NS>(sums + lr * T::NP, row0 + lr, i, inv_k, alpha_pre, alpha_post, alpha_res,
                   bsh, bsh + NS, bsh + 2 * NS, r_out, H);
}

}  // namespace

// Process-wide call epoch, from a start that differs between runs.
unsigned long long next_call_epoch() {
  static std::atomic<unsigned long long> counter{
      (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull};
  unsigned long long e;
  do {
    e = counter.fetch_add(1, std::memory_order_relaxed);
  } while (e == 0);
  return e;
}

namespace {

template <int NS, bool FP8X, bool P32>
hipError_t launch_small_n(const SmallPlan &p, int64_t B, int64_t C, const void *X,
                          const void *phi, float ap, float aq, float ar, const float *bp,
                          const float *bq, const float *br, float *logits, float *r, float *H,
                          void *ws_base, hipStream_t st) {
  char *base = static_cast<char *>(ws_base);
  const dim3 grid((uint32_t)p.row_tiles, (uint32_t)p.split);
  const float inv_k = (float)(1.0 / (double)(NS * C));
  coeffs_small_kernel<NS, FP8X, P32><<<grid, 256, 0, st>>>(
      static_cast<const uint8_t *>(X), phi, (int)B,
      (int)(NS * C), p.split, inv_k, ap, aq, ar, bp, bq, br, logits, r, H,
      reinterpret_cast<float *>(base), reinterpret_cast<unsigned long long *>(base + p.ctr_offset),
      next_call_epoch());
  return hipGetLastError();
}

}  // namespace

SmallPlan plan_coeffs_small(int64_t B, int n, int64_t C) {
  SmallPlan p;
  const int64_t N = (int64_t)n * n + 2 * n, K = (int64_t)n * C;
  int64_t ks = 0;
  switch (n) {
    case 1: ks = kSmallKSlice<1>(); break;
    case 2: ks = kSmallKSlice<2>(); break;
    case 4: ks = kSmallKSlice<4>(); break;
    default: ks = kSmallKSlice<8>(); break;
  }
  p.kslice = ks;
  p.split = (int)((K + ks - 1) / ks);
  p.row_tiles = (B + 15) / 16;
  p.partial_bytes = (size_t)p.split * (size_t)B * (size_t)(N + 1) * sizeof(float);
  p.ctr_offset = (p.partial_bytes + 255) & ~(size_t)255;
  p.total_bytes = p.ctr_offset + (size_t)p.row_tiles * (size_t)p.split * 8;
  return p;
}

bool use_coeffs_small(int64_t B, int n, int64_t C) {
  const int64_t max_b = tune(kTuneSmallMaxB) >= 0 ? tune(kTuneSmallMaxB) : kSmallMaxB;  // 0: never
  return B <= max_b && plan_coeffs_small(B, n, C).split <= kSmallMaxSplit;
}

template <bool FP8X, bool P32>
hipError_t launch_small_x(const SmallPlan &p, int n, int64_t B, int64_t C, const void *X,
                          const void *phi, float ap, float aq, float ar, const float *bp,
                          const float *bq, const float *br, float *logits, float *r, float *H,
                          void *ws, hipStream_t st) {
  switch (n) {
    case 1: return launch_small_n<1, FP8X, P32>(p, B, C, X, phi, ap, aq, ar, bp, bq, br, logits, r, H, ws, st);
    case 2: return launch_small_n<2, FP8X, P32>(p, B, C, X, phi, ap, aq, ar, bp, bq, br, logits, r, H, ws, st);
    case 4: return launch_small_n<4, FP8X, P32>(p, B, C, X, phi, ap, aq, ar, bp, bq, br, logits, r, H, ws, st);
    case 8: return launch_small_n<8, FP8X, P32>(p, B, C, X, phi, ap, aq, ar, bp, bq, br, logits, r, H, ws, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_coeffs_small(const SmallPlan &p, int n, bool fp8_x, int64_t B, int64_t C,
                               const void *X, const void *phi, float ap, float aq, float ar,
                               const float *bp, const float *bq, const float *br, float *logits,
                               float *r, float *H, void *ws, hipStream_t st, bool phi32) {
  if (phi32)  // fp32 phi is offered with bf16 X only
    return fp8_x ? hipErrorInvalidValue
                 : launch_small_x<false, true>(p, n, B, C, X, phi, ap, aq, ar, bp, bq, br, logits, r, H, ws, st);
  return fp8_x ? launch_small_x<true, false>(p, n, B, C, X, phi, ap, aq, ar, bp, bq, br, logits, r, H, ws, st)
               : launch_small_x<false, false>(p, n, B, C, X, phi, ap, aq, ar, bp, bq, br, logits, r, H, ws, st);
}

}  // namespace mhc
