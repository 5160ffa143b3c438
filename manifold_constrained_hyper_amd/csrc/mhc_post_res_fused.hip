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
// A workgroup is 16 waves and owns a tile of 16 rows; it walks the hidden
// dimension in steps of 512 channels (its K-slice: a channel range of all n
// streams).  Per step:
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
//            v_mfma_f32_16x16x32_bf16 plus the Gram block for sum of squares.
// The loads of step c+1 are issued before the product of step c.  At the end
// the 16 waves' accumulators are summed through LDS in wave order (fixed:
// deterministic) into the workspace partials fp32 [S, B, N+1], which the
// combine kernel turns into the next layer's logits, r and H.
//
// The apply arithmetic is that of post_res_kernel (fp32 FMA chain from
// H_post * F_out, one round-to-nearest-even to bf16), so X_{t+1} is bitwise
// what the stand-alone apply writes, and the product consumes those rounded
// values, exactly what a separate product pass would read back.
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

constexpr int kStepCh = 512;  // channels per step: 64 lanes x 8

template <int NS>
struct FusedTile {
  static constexpr int N = NS * NS + 2 * NS;
  static constexpr int NP = N + 1;
  static constexpr int NB = (N + 15) / 16;
  static constexpr int ROW_BYTES = NS * kStepCh * 2;   // one tile row in LDS
  static constexpr int LDS_BYTES = 16 * ROW_BYTES;     // 64 KiB at n=4, 128 KiB at n=8
  static constexpr int KSTEPS = 16 * NS;               // 32-channel MFMA steps per step
  static constexpr int KPW = KSTEPS / 16;              // ... per wave (= NS)
  static constexpr int KB = NS >= 8 ? 2 : (KPW < 4 ? KPW : 4);  // k-steps whose B operands are held at once
  static_assert(16 * 16 * NP * 4 <= LDS_BYTES, "reduction scratch fits in the tile buffer");
};

template <int NS>
__global__ __launch_bounds__(1024) void post_res_next_kernel(
    const uint16_t *__restrict__ X, const uint16_t *__restrict__ F, const float *__restrict__ H,
    uint16_t *__restrict__ Y, const uint16_t *__restrict__ phip, float *__restrict__ ws, int B,
    int C, int cw) {
  using T = FusedTile<NS>;
  __shared__ __attribute__((aligned(1024))) char lds[T::LDS_BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int s = blockIdx.y;
  const int c_begin = s * cw;
  const int c_end = min(C, c_begin + cw);
  const int row0 = blockIdx.x * 16;

  // apply role: wave `wave` owns tile row `wave`
  const int my_row = row0 + wave;
  const bool live = my_row < B;
  const int rr = uniform(min(my_row, B - 1));
  const uint16_t *xr = X + (size_t)rr * NS * C;
  const uint16_t *fr = F + (size_t)rr * C;
  uint16_t *yr = Y + (size_t)rr * NS * C;
  float hpost[NS], hres[NS][NS];
  {
    const float *h = H + (size_t)rr * T::N;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      hpost[i] = h[NS + i];
#pragma unroll
      for (int j = 0; j < NS; ++j) hres[i][j] = h[2 * NS + i * NS + j];
    }
  }
  char *my_lds_row = lds + wave * T::ROW_BYTES;
  const int wslot = (lane ^ (wave & 15)) * 16;  // swizzled 16-byte slot of this lane

  f32x4 acc[T::NB], gram;
  gram = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < T::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads of one step.  Lanes past the range read an in-range address
  // instead (their values are never stored and enter the tile as zeros), so
  // every wave issues the same loads on every step and the waits before the
  // product only ever cover the operand loads, never the prefetch.
  u32x4 xv[NS], fv;
  auto load_step = [&](int c0) {
    const int c = min(c0 + 8 * lane, c_end - 8);
#pragma unroll
    for (int j = 0; j < NS; ++j)
      xv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + (size_t)j * C + c));
    fv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(fr + c));
  };

  load_step(c_begin);
  for (int c0 = c_begin; c0 < c_end; c0 += kStepCh) {
    const int c = c0 + 8 * lane;
    // apply (row `wave`, channels c .. c+7 of every stream)
    u32x4 out[NS];
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
    const bool in_range = c < c_end;
    if (live && in_range) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
        __builtin_nontemporal_store(out[i], reinterpret_cast<u32x4 *>(yr + (size_t)i * C + c));
    }
    // B operands of this wave's k-steps (global, L2-resident), issued before
    // the prefetch so that waiting for them never waits for the prefetch.
    // They are held in groups of KB k-steps (all of them for n <= 4; for n = 8
    // the later groups are loaded after the earlier ones are consumed).
    bf16x8 b[T::KB][T::NB];
    auto load_b = [&](int q0) {
#pragma unroll
      for (int q = 0; q < T::KB; ++q) {
        const int ks = wave * T::KPW + q0 + q;       // 0 .. 16*NS-1 within the step
        const int i = ks >> 4, t = ks & 15;          // stream, 32-channel sub-step
        const int cs = c0 + 32 * t;
        const int kstep = (i * C + min(cs, C - 32)) >> 5;  // clamped in range; such steps add zero
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
          b[q][nb] = __builtin_bit_cast(bf16x8, load16(phip + ((size_t)(kstep * T::NB + nb) * 64 + lane) * 8));
      }
    };
    load_b(0);
    __syncthreads();  // the previous step's product is done reading the tile
#pragma unroll
    for (int i = 0; i < NS; ++i)
      *reinterpret_cast<u32x4 *>(my_lds_row + i * (kStepCh * 2) + wslot) =
          in_range ? out[i] : u32x4{0u, 0u, 0u, 0u};
    load_step(min(c0 + kStepCh, c_end - 8));  // prefetch the next step (a harmless reload after the last)
    __syncthreads();  // the tile is complete

    // k-steps past the range read zeros from the tile (those lanes stored
    // zeros), so they add nothing; no branch is needed.
#pragma unroll
    for (int q0 = 0; q0 < T::KPW; q0 += T::KB) {
      if (q0 > 0) load_b(q0);
#pragma unroll
      for (int q = 0; q < T::KB; ++q) {
        const int ks = wave * T::KPW + q0 + q;
        const int i = ks >> 4, t = ks & 15;
        const int piece = (4 * t + g) ^ m;
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(lds + m * T::ROW_BYTES + i * (kStepCh * 2) + piece * 16);
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[q][nb], acc[nb], 0, 0, 0);
        gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, gram, 0, 0, 0);
      }
    }
  }

  // Reduce the 16 waves' accumulators through LDS, in wave order.
  __syncthreads();
  float *red = reinterpret_cast<float *>(lds);  // [16 waves][16 rows][NP]
#pragma unroll
  for (int nb = 0; nb < T::NB; ++nb) {
    const int col = nb * 16 + m;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (col < T::N) red[(wave * 16 + 4 * g + v) * T::NP + col] = acc[nb][v];
  }
  if (g == (m >> 2)) red[(wave * 16 + m) * T::NP + T::N] = gram[m & 3];
  __syncthreads();
  float *wsl = ws + (size_t)s * B * T::NP;
  for (int e = tid; e < 16 * T::NP; e += 1024) {
    const int r = e / T::NP, col = e - r * T::NP;
    float a = 0.f;
    for (int w = 0; w < 16; ++w) a += red[(w * 16 + r) * T::NP + col];
    if (row0 + r < B) wsl[(size_t)(row0 + r) * T::NP + col] = a;
  }
}

}  // namespace

template <int NS>
hipError_t launch_post_res_next_typed(int64_t B, int64_t C, int cw, int split, const void *X,
                                      const void *F, const float *H, void *Y, const void *phip,
                                      float *ws, hipStream_t st) {
  const dim3 grid((uint32_t)((B + 15) / 16), (uint32_t)split);
  post_res_next_kernel<NS><<<grid, 1024, 0, st>>>(
      static_cast<const uint16_t *>(X), static_cast<const uint16_t *>(F), H,
      static_cast<uint16_t *>(Y), static_cast<const uint16_t *>(phip), ws, (int)B, (int)C, cw);
  return hipGetLastError();
}

FusedPlan plan_post_res_next(int64_t B, int n, int64_t C) {
  FusedPlan p;
  const int64_t N = (int64_t)n * n + 2 * n, NB = (N + 15) / 16, K = (int64_t)n * C;
  p.row_tiles = (B + 15) / 16;
  // One slice of the whole hidden size when there are enough row tiles to
  // fill the machine (one 16-wave workgroup per CU at a time); otherwise
  // split the channels so that about 512 workgroups exist.
  const int64_t steps = (C + kStepCh - 1) / kStepCh;
  int64_t want = (512 + p.row_tiles - 1) / p.row_tiles;
  if (want < 1) want = 1;
  if (want > steps) want = steps;
  p.cw = (int)(((steps + want - 1) / want) * kStepCh);
  p.split = (int)((C + p.cw - 1) / p.cw);
  p.partial_bytes = (size_t)p.split * (size_t)B * (size_t)(N + 1) * sizeof(float);
  p.ksteps = (K + 31) / 32;
  p.phip_offset = (p.partial_bytes + 1023) & ~(size_t)1023;
  p.phip_bytes = (size_t)p.ksteps * (size_t)NB * 1024;
  p.zero_offset = p.phip_offset + p.phip_bytes;
  p.total_bytes = p.zero_offset + 256;
  return p;
}

hipError_t launch_post_res_next(const FusedPlan &p, int n, int64_t B, int64_t C, const void *X,
                                const void *F, const float *H, void *Y, const void *phi_next,
                                void *ws_base, hipStream_t st) {
  char *base = static_cast<char *>(ws_base);
  void *phip = base + p.phip_offset;
  hipError_t e = launch_pack_phi(n, (int64_t)n * C, p.ksteps, phi_next, phip, base + p.zero_offset, st);
  if (e != hipSuccess) return e;
  float *ws = reinterpret_cast<float *>(base);
  switch (n) {
    case 1: return launch_post_res_next_typed<1>(B, C, p.cw, p.split, X, F, H, Y, phip, ws, st);
    case 2: return launch_post_res_next_typed<2>(B, C, p.cw, p.split, X, F, H, Y, phip, ws, st);
    case 4: return launch_post_res_next_typed<4>(B, C, p.cw, p.split, X, F, H, Y, phip, ws, st);
    case 8: return launch_post_res_next_typed<8>(B, C, p.cw, p.split, X, F, H, Y, phip, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhc
