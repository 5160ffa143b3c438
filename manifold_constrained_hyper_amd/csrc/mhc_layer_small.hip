// Single-slice layer calls in one kernel: mhc_post_res_coeffs_pre and
// mhc_coeffs_pre in bf16 for n in {1, 2, 4}, the small-B sizes of mhc_coeffs
// (up to 256 rows), when a row's K = n*C channels fit one 1024-channel slice
// (C <= 1024/n).
//
// [mHC-cutile] (page "mHC 算法分析 & cutile 高效实现") section 2.5 (third
// step) forms X_{t+1} from X_t, F_out and H; sections 2.1-2.4 form the next
// layer's logits, r and H from X_{t+1}; section 2.5 (first step) then needs
// F_pre = sum_i H_pre[i] X_{t+1}[i].  Section 3.2 notes that at these sizes
// the steps are bound by launches and latency, not by bytes.  When all of a
// row's channels fit one workgroup, one workgroup per 16-row tile does the
// whole layer for its rows, with no hand-off between workgroups:
//
//   apply    lane (m, g) of wave w takes row m of the tile and channels
//            32 ts + 8 g .. +7 of every stream for the wave's sub-blocks ts;
//            it computes X_{t+1} exactly as post_res_kernel (the row's own
//            coefficients, loaded per lane) and stores it;
//   product  those bf16 values are, as they stand in the lanes, the A
//            operands of v_mfma_f32_16x16x32_bf16 (row m, k = 8 g .. +7 of the
//            32-channel k-step of one stream); the B operands come from phi,
//            transposed into LDS on the way in (one column's channels
//            contiguous, so an operand is one 16-byte LDS read); the Gram
//            block gives the sum of squares;
//   sums     the four waves' partial sums, added in wave order;
//   F_pre    H_pre of the tile's rows from those sums (pre_gate, as the
//            finish does), then F_pre for the lane's channels from the
//            X_{t+1} values still in its lanes, exactly as pre_kernel would;
//   finish   finish_row for the tile's rows: logits, r and H.  The biases are
//            staged in LDS at the start, so nothing after the product waits
//            on global memory.
//
// With several slices the workgroups of a row tile would have to exchange
// their partial sums through memory within the launch; measured at 64 rows
// that exchange costs more than the launches it saves, so those shapes keep
// the split-K coefficient kernel and the separate apply and pre-mix.  The
// product-only mode (mhc_coeffs_pre) skips the apply and multiplies X_t.
#include "mhc_device.h"
#include "mhc_finish.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

template <int NS>
struct LayerTile {
  static constexpr int N = NS * NS + 2 * NS;
  static constexpr int NP = N + 1;
  static constexpr int NB = (N + 15) / 16;
  static constexpr int RS = NB * 16 + 1;  // reduction row stride; Gram sum at NB*16
  static constexpr int CW = 1024 / NS;    // channels per stream (K = 1024 at most)
  static constexpr int LDK = CW + 8;      // LDS row of one (stream, column): CW channels + pad
  static constexpr int TSW = CW / 32 / 4; // 32-channel sub-blocks per wave
  static constexpr int G = N % 2 == 0 ? 4 : 8;   // channels per phi staging group (G*N*2 % 16 == 0)
  static constexpr int GP = G * N / 8;            // 16-byte pieces per group
  static constexpr int GPS = CW / G;              // groups per stream
  static constexpr int NG = NS * GPS;             // groups (one per thread at most)
  static_assert(NG <= 256 && (G * N) % 8 == 0, "phi staging groups");
};

// The part both kernels share, for the workgroup's 16-row tile (rows from
// row0) and channels c0 .. c0 + CW-1 of every stream: loads, phi staged
// transposed in LDS, the apply (APPLY: X_{t+1} into xn and stored to Y;
// otherwise xn = X_t), the product and the four waves' partial sums in red
// (row r, column col at red[(w*16 + r)*RS + col], the Gram sum at column
// NB*16).  Ends with a barrier.
template <int NS, bool APPLY>
__device__ __forceinline__ void layer_front(const uint16_t *__restrict__ X, const uint16_t *__restrict__ F,
                                            const float *__restrict__ H, uint16_t *__restrict__ Y,
                                            const uint16_t *__restrict__ phi, int B, int C, int row0, int c0,
                                            uint16_t *phs, float *red, u32x4 (&xn)[LayerTile<NS>::TSW][NS],
                                            int (&cl)[LayerTile<NS>::TSW]) {
  using T = LayerTile<NS>;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int row = row0 + m;
  const int rr = min(row, B - 1);  // rows past B repeat row B-1 (nothing of theirs is stored)
  const int K = NS * C;
  const bool live = row < B;

  // ---- loads: this lane's X (and F_out, coefficients), then phi
  u32x4 xv[T::TSW][NS];
  [[maybe_unused]] u32x4 fv[T::TSW];
#pragma unroll
  for (int q = 0; q < T::TSW; ++q) {
    const int c = c0 + 32 * (wave * T::TSW + q) + 8 * g;
    cl[q] = c;
    const int cc = min(c, C - 8);
#pragma unroll
    for (int i = 0; i < NS; ++i) xv[q][i] = load16(X + ((size_t)rr * K + (size_t)i * C + cc));
    if constexpr (APPLY) fv[q] = load16(F + ((size_t)rr * C + cc));
  }
  [[maybe_unused]] float hpost[NS], hres[NS][NS];
  if constexpr (APPLY) {
    const float *h = H + (size_t)rr * T::N;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      hpost[i] = h[NS + i];
#pragma unroll
      for (int j = 0; j < NS; ++j) hres[i][j] = h[2 * NS + i * NS + j];
    }
  }
  {
    // phi rows i*C + c0 .. i*C + c0 + CW-1 of each stream, transposed into
    // LDS: element (channel c0 + k, column col) of stream i goes to
    // phs[(i*N + col)*LDK + k], zero for c0 + k >= C.  Thread t takes group t:
    // G consecutive channels of one stream (G*N elements, GP contiguous
    // 16-byte pieces), and writes each column's G channels with one 8- or
    // 16-byte LDS store.  C % 8 == 0, so a group lies wholly below C or wholly
    // past it.
    const int gi = tid;
    const int i = min(gi / T::GPS, NS - 1), k0 = (gi - i * T::GPS) * T::G;
    const bool gv = gi < T::NG && c0 + k0 < C;
    const char *src = reinterpret_cast<const char *>(phi + ((size_t)i * C + c0 + (gv ? k0 : 0)) * T::N);
    u32x4 v[T::GP];
#pragma unroll
    for (int q = 0; q < T::GP; ++q) v[q] = load16(src + 16 * q);
    if (gi < T::NG) {
#pragma unroll
      for (int col = 0; col < T::N; ++col) {
        uint32_t w[T::G / 2];
#pragma unroll
        for (int t = 0; t < T::G / 2; ++t) {
          const int fl = (2 * t) * T::N + col, fh = fl + T::N;  // elements (k0+2t, col), (k0+2t+1, col)
          const uint32_t lo = (v[fl >> 3][(fl & 7) >> 1] >> (16 * (fl & 1))) & 0xffffu;
          const uint32_t hi = (v[fh >> 3][(fh & 7) >> 1] >> (16 * (fh & 1))) & 0xffffu;
          w[t] = gv ? (lo | (hi << 16)) : 0u;
        }
        uint16_t *dst = phs + (i * T::N + col) * T::LDK + k0;
        if constexpr (T::G == 4) {
          *reinterpret_cast<u32x2 *>(dst) = u32x2{w[0], w[1]};
        } else {
          *reinterpret_cast<u32x4 *>(dst) = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
    }
  }

  // ---- apply (post_res_kernel's arithmetic) and store X_{t+1}
#pragma unroll
  for (int q = 0; q < T::TSW; ++q) {
    if constexpr (APPLY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f0 = bf16_lo(fv[q][w]), f1 = bf16_hi(fv[q][w]);
        float x0[NS], x1[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          x0[j] = bf16_lo(xv[q][j][w]);
          x1[j] = bf16_hi(xv[q][j][w]);
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          float a0 = hpost[i] * f0, a1 = hpost[i] * f1;
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            a0 = fmaf(hres[i][j], x0[j], a0);
            a1 = fmaf(hres[i][j], x1[j], a1);
          }
          xn[q][i][w] = pack_bf16x2(a0, a1);
        }
      }
      if (live && cl[q] < C) {
#pragma unroll
        for (int i = 0; i < NS; ++i) store16_plain(Y + ((size_t)row * K + (size_t)i * C + cl[q]), xn[q][i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NS; ++i) xn[q][i] = xv[q][i];
    }
  }
  __syncthreads();  // phs and bsh complete

  // ---- product: k-step (stream i, sub-block ts) with this lane's values
  f32x4 acc[T::NB], gram = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < T::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < T::TSW; ++q) {
    const int ts = wave * T::TSW + q;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, cl[q] < C ? xn[q][i] : u32x4{0u, 0u, 0u, 0u});
      const int kk = 32 * ts + 8 * g;  // channel within the slice
#pragma unroll
      for (int nb = 0; nb < T::NB; ++nb) {
        const int col = nb * 16 + m;
        const u32x4 w = col < T::N ? *reinterpret_cast<const u32x4 *>(phs + (i * T::N + col) * T::LDK + kk)
                                   : u32x4{0u, 0u, 0u, 0u};
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, w), acc[nb], 0, 0, 0);
      }
      gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, gram, 0, 0, 0);
    }
  }
  {
    float *rw = red + wave * 16 * T::RS;
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) rw[(4 * g + v) * T::RS + nb * 16 + m] = acc[nb][v];
    if (g == (m >> 2)) rw[m * T::RS + T::NB * 16] = gram[m & 3];
  }
  __syncthreads();
}

template <int NS, bool APPLY>
__global__ __launch_bounds__(256) void layer_small_kernel(
    const uint16_t *__restrict__ X, const uint16_t *__restrict__ F, const float *__restrict__ H,
    uint16_t *__restrict__ Y, const uint16_t *__restrict__ phi, int B, int C, float inv_k,
    float alpha_pre, float alpha_post, float alpha_res, const float *__restrict__ b_pre,
    const float *__restrict__ b_post, const float *__restrict__ b_res, float *__restrict__ logits,
    float *__restrict__ r_out, float *__restrict__ Hn, uint16_t *__restrict__ F_pre) {
  using T = LayerTile<NS>;
  __shared__ __attribute__((aligned(16))) uint16_t phs[NS * T::N * T::LDK];  // [stream][column][channel]
  __shared__ float red[4 * 16 * T::RS];
  __shared__ float sums[16 * T::NP];
  __shared__ float hpre[16 * NS];
  __shared__ float bsh[T::N];  // b_pre, b_post, b_res

  const int tid = threadIdx.x;
  const int m = tid & 15;
  const int row0 = blockIdx.x * 16;
  const int row = row0 + m;
  const bool live = row < B;
  if (tid < T::N) bsh[tid] = tid < NS ? b_pre[tid] : (tid < 2 * NS ? b_post[tid - NS] : b_res[tid - 2 * NS]);

  u32x4 xn[T::TSW][NS];
  int cl[T::TSW];
  layer_front<NS, APPLY>(X, F, H, Y, phi, B, C, row0, 0, phs, red, xn, cl);

  // ---- sums: the four waves' partials, added in wave order
  for (int e = tid; e < 16 * T::NP; e += 256) {
    const int r = e / T::NP, col = e - r * T::NP;
    const int rcol = col < T::N ? col : T::NB * 16;
    sums[e] = ((red[(0 * 16 + r) * T::RS + rcol] + red[(1 * 16 + r) * T::RS + rcol]) +
               red[(2 * 16 + r) * T::RS + rcol]) + red[(3 * 16 + r) * T::RS + rcol];
  }
  __syncthreads();

  // ---- H_pre of the tile's rows (the finish's formula: equal sums, equal bits)
  if (tid < 16 * NS) {
    const int r = tid / NS, i = tid - r * NS;
    const float inv_r = recip_exact(row_rms(sums[r * T::NP + T::N], inv_k));
    hpre[tid] = pre_gate(sums[r * T::NP + i], inv_r, alpha_pre, bsh[i]);
  }
  __syncthreads();

  // ---- F_pre for this lane's channels (pre_kernel's arithmetic)
#pragma unroll
  for (int q = 0; q < T::TSW; ++q) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        a0 = fmaf(hpre[m * NS + j], bf16_lo(xn[q][j][w]), a0);
        a1 = fmaf(hpre[m * NS + j], bf16_hi(xn[q][j][w]), a1);
      }
      o[w] = pack_bf16x2(a0, a1);
    }
    if (live && cl[q] < C) store16_plain(F_pre + ((size_t)row * C + cl[q]), o);
  }

  // ---- finish: logits, r and H of the tile's rows
  const int rows = min(16, B - row0);
  for (int e = tid; e < rows * T::N; e += 256) {
    const int r = e / T::N, col = e - r * T::N;
    logits[(size_t)(row0 + r) * T::N + col] = sums[r * T::NP + col];
  }
  const int lr = tid / NS, i = tid % NS;
  if (lr < rows)
    finish_row<NS>(sums + lr * T::NP, row0 + lr, i, inv_k, alpha_pre, alpha_post, alpha_res, bsh, bsh + NS,
                   bsh + 2 * NS, r_out, Hn);
}

// mhc_post_res_coeffs at the small-B sizes, split over K: workgroup (tile,
// s) runs layer_front for channels s*CW .. s*CW + CW-1 of every stream
// (X_{t+1} stored), writes its [16, N+1] partial to the workspace
// [S, B, N+1] with agent-scope stores, waits for them, then writes the call's
// epoch into its flag (one per tile and slice) and waits for that too.  Wave
// 0 reads the tile's S flags; a workgroup that finds all of them carrying the
// epoch adds the S partials in slice order 0..S-1, writes the logits, clears
// the flags (so a replay of the same launch starts clean) and runs the finish.
// Every workgroup's flag is complete before it reads the others', so the last
// to arrive always sees all flags, and two that both see them write the same
// bits.  No workgroup waits for another.  With one slice the workgroup
// finishes from LDS.
template <int NS>
__global__ __launch_bounds__(256) void apply_coeffs_small_kernel(
    const uint16_t *__restrict__ X, const uint16_t *__restrict__ F, const float *__restrict__ H,
    uint16_t *__restrict__ Y, const uint16_t *__restrict__ phi, int B, int C, int S, float inv_k,
    float alpha_pre, float alpha_post, float alpha_res, const float *__restrict__ b_pre,
    const float *__restrict__ b_post, const float *__restrict__ b_res, float *__restrict__ logits,
    float *__restrict__ r_out, float *__restrict__ Hn, float *__restrict__ ws,
    unsigned long long *__restrict__ flags, unsigned long long epoch) {
  using T = LayerTile<NS>;
  constexpr int EPT = (16 * T::NP + 255) / 256;  // tile sums per thread in the combine
  constexpr int kCombineBatch = combine_batch(EPT);
  __shared__ __attribute__((aligned(16))) uint16_t phs[NS * T::N * T::LDK];  // [stream][column][channel]
  __shared__ float red[4 * 16 * T::RS];
  __shared__ float sums[16 * T::NP];
  __shared__ float bsh[T::N];  // b_pre, b_post, b_res
  __shared__ int is_last;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int tile = blockIdx.x, s = blockIdx.y;
  const int row0 = tile * 16;
  const int rows = min(16, B - row0);
  if (tid < T::N) bsh[tid] = tid < NS ? b_pre[tid] : (tid < 2 * NS ? b_post[tid - NS] : b_res[tid - 2 * NS]);

  u32x4 xn[T::TSW][NS];
  int cl[T::TSW];
  layer_front<NS, true>(X, F, H, Y, phi, B, C, row0, s * T::CW, phs, red, xn, cl);

  const size_t slice = (size_t)B * T::NP;
  if (S == 1) {
    for (int e = tid; e < rows * T::NP; e += 256) {
      const int r = e / T::NP, col = e - r * T::NP;
      const int rcol = col < T::N ? col : T::NB * 16;
      const float v = ((red[(0 * 16 + r) * T::RS + rcol] + red[(1 * 16 + r) * T::RS + rcol]) +
                       red[(2 * 16 + r) * T::RS + rcol]) + red[(3 * 16 + r) * T::RS + rcol];
      sums[e] = v;
      if (col < T::N) logits[(size_t)(row0 + r) * T::N + col] = v;
    }
  } else {
    for (int e = tid; e < 16 * T::NP; e += 256) {
      const int r = e / T::NP, col = e - r * T::NP;
      const int rcol = col < T::N ? col : T::NB * 16;
      const float v = ((red[(0 * 16 + r) * T::RS + rcol] + red[(1 * 16 + r) * T::RS + rcol]) +
                       red[(2 * 16 + r) * T::RS + rcol]) + red[(3 * 16 + r) * T::RS + rcol];
      if (row0 + r < B)
        __hip_atomic_store(ws + (size_t)s * slice + (size_t)(row0 + r) * T::NP + col, v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
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

    // Last slice of the tile to arrive: the S partials in slice order (a
    // thread's loads for kCombineBatch slices issued before any is added:
    // one memory round trip up to 32 slices at n <= 4).
    const float *base = ws + (size_t)row0 * T::NP;
    const int nel = rows * T::NP;
    float tot[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) tot[q] = 0.f;
    for (int s0 = 0; s0 < S; s0 += kCombineBatch) {
      float v[kCombineBatch][EPT];
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j)
#pragma unroll
        for (int q = 0; q < EPT; ++q)
          v[j][q] = __hip_atomic_load(base + (size_t)min(s0 + j, S - 1) * slice + min(tid + 256 * q, nel - 1),
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j)
#pragma unroll
        for (int q = 0; q < EPT; ++q)
          if (s0 + j < S) tot[q] += v[j][q];
    }
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = tid + 256 * q;
      if (e < nel) {
        sums[e] = tot[q];
        const int r = e / T::NP, col = e - r * T::NP;
        if (col < T::N) logits[(size_t)(row0 + r) * T::N + col] = tot[q];
      }
    }
    // Every slice has arrived, so no workgroup reads the tile's flags any more.
    if (wave == 0 && lane < S)
      __hip_atomic_store(tflags + lane, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const int lr = tid / NS, i = tid % NS;
  if (lr < rows)
    finish_row<NS>(sums + lr * T::NP, row0 + lr, i, inv_k, alpha_pre, alpha_post, alpha_res, bsh, bsh + NS,
                   bsh + 2 * NS, r_out, Hn);
}

template <int NS>
hipError_t launch_apply_coeffs_n(const SmallPlan &p, int64_t B, int64_t C, const void *X, const void *F,
                                 const float *H, void *Y, const void *phi, float ap, float aq, float ar,
                                 const float *bp, const float *bq, const float *br, float *logits, float *r,
                                 float *Hn, void *ws_base, hipStream_t st) {
  char *base = static_cast<char *>(ws_base);
  const float inv_k = (float)(1.0 / (double)(NS * C));
  apply_coeffs_small_kernel<NS><<<dim3((uint32_t)p.row_tiles, (uint32_t)p.split), 256, 0, st>>>(
      static_cast<const uint16_t *>(X), static_cast<const uint16_t *>(F), H, static_cast<uint16_t *>(Y),
      static_cast<const uint16_t *>(phi), (int)B, (int)C, p.split, inv_k, ap, aq, ar, bp, bq, br, logits, r, Hn,
      reinterpret_cast<float *>(base), reinterpret_cast<unsigned long long *>(base + p.ctr_offset),
      next_call_epoch());
  return hipGetLastError();
}

template <int NS, bool APPLY>
hipError_t launch_layer_n(int64_t B, int64_t C, const void *X, const void *F, const float *H, void *Y,
                          const void *phi, float ap, float aq, float ar, const float *bp, const float *bq,
                          const float *br, float *logits, float *r, float *Hn, void *F_pre, hipStream_t st) {
  const float inv_k = (float)(1.0 / (double)(NS * C));
  layer_small_kernel<NS, APPLY><<<dim3((uint32_t)((B + 15) / 16)), 256, 0, st>>>(
      static_cast<const uint16_t *>(X), static_cast<const uint16_t *>(F), H, static_cast<uint16_t *>(Y),
      static_cast<const uint16_t *>(phi), (int)B, (int)C, inv_k, ap, aq, ar, bp, bq, br, logits, r, Hn,
      static_cast<uint16_t *>(F_pre));
  return hipGetLastError();
}

}  // namespace

bool layer_small_fits(int64_t B, int n, int64_t C) {
  if (n != 1 && n != 2 && n != 4) return false;
  return B >= 1 && C >= 8 && C % 8 == 0 && C * n <= 1024 && use_coeffs_small(B, n, C);
}

bool apply_coeffs_small_fits(int64_t B, int n, int64_t C) {
  if (n != 1 && n != 2 && n != 4) return false;
  return B >= 1 && C >= 8 && C % 8 == 0 && use_coeffs_small(B, n, C);
}

hipError_t launch_apply_coeffs_small(const SmallPlan &p, int n, int64_t B, int64_t C, const void *X,
                                     const void *F, const float *H, void *Y, const void *phi, float ap, float aq,
                                     float ar, const float *bp, const float *bq, const float *br, float *logits,
                                     float *r, float *Hn, void *ws, hipStream_t st) {
  if (!apply_coeffs_small_fits(B, n, C) || p.split != (int)((C * n + 1023) / 1024)) return hipErrorInvalidValue;
  switch (n) {
    case 1: return launch_apply_coeffs_n<1>(p, B, C, X, F, H, Y, phi, ap, aq, ar, bp, bq, br, logits, r, Hn, ws, st);
    case 2: return launch_apply_coeffs_n<2>(p, B, C, X, F, H, Y, phi, ap, aq, ar, bp, bq, br, logits, r, Hn, ws, st);
    case 4: return launch_apply_coeffs_n<4>(p, B, C, X, F, H, Y, phi, ap, aq, ar, bp, bq, br, logits, r, Hn, ws, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_layer_small(int n, bool apply, int64_t B, int64_t C, const void *X, const void *F,
                              const float *H, void *Y, const void *phi, float ap, float aq, float ar,
                              const float *bp, const float *bq, const float *br, float *logits, float *r,
                              float *Hn, void *F_pre, hipStream_t st) {
  if (!layer_small_fits(B, n, C)) return hipErrorInvalidValue;
#define MHC_LAYER_CASE(NSV)                                                                                   \
  case NSV:                                                                                                   \
    return apply ? launch_layer_n<NSV, true>(B, C, X, F, H, Y, phi, ap, aq, ar, bp, bq, br, logits, r, Hn,    \
                                             F_pre, st)                                                       \
                 : launch_layer_n<NSV, false>(B, C, X, F, H, Y, phi, ap, aq, ar, bp, bq, br, logits, r, Hn,   \
                                              F_pre, st);
  switch (n) {
    MHC_LAYER_CASE(1)
    MHC_LAYER_CASE(2)
    MHC_LAYER_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef MHC_LAYER_CASE
}

}  // namespace mhc
