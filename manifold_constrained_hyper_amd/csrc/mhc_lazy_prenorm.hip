// Lazy Pre-Norm GEMM: C = rmsnorm(A) @ W^T in one kernel.
//
// [FreeNorm] (the PyTorch blog "Towards Free Normalization: Fusing
// Normalization into GEMM and Attention Kernels"), section 2: with rmsnorm
// without an affine weight, rmsnorm(A) = diag(rstd) A, so
// rmsnorm(A) @ B = diag(rstd) (A @ B): the GEMM runs on the raw A, the row
// sums of squares are accumulated in the same k-loop, and each output row is
// scaled by rstd = rsqrt(sum(A^2)/K + eps) at the end.  B is passed as its
// transpose W [N, K] (a linear layer's weight), so both operands are
// K-contiguous rows.
//
// gfx950 design (the page's kernel is TLX/Blackwell; this is written for
// CDNA4):
//  * workgroup tile 256 x 256 of C, 4 waves, each 128 x 128 (8 x 8 blocks of
//    v_mfma_f32_16x16x32_bf16: 256 accumulator registers per wave, one wave
//    per SIMD);
//  * A and W tiles move to LDS by direct-to-LDS loads (global_load_lds_dwordx4,
//    each instruction 1 KiB = 8 rows of a 64-k chunk), two stages of 64 KiB;
//    within a 128-byte row the 16-byte pieces are XOR-swizzled by
//    ((row >> 1) & 7), which makes the operand ds_read_b128 of 16 rows
//    bank-conflict-free;
//  * each block computes C^T = W A^T (W as the MFMA A operand), so a lane ends
//    with 4 consecutive output columns of one row: the epilogue scales them
//    by that row's rstd and stores 8 bytes;
//  * the row sums of squares run on the vector unit beside the matrix core:
//    thread t adds the squares of row t of every A chunk in LDS (the matrix
//    core's accumulators fill the 256 AGPRs, so a Gram block there would
//    spill);
//  * tiles are walked in groups of 16 tile rows (so the ~256 resident
//    workgroups share A and W tiles in L2 / MALL), each XCD taking a
//    contiguous run of the order.
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTM = 256, kTN = 256;  // workgroup tile
constexpr int kKC = 64;              // k per chunk
constexpr int kRowBytes = kKC * 2;   // 128 bytes: 8 pieces of 16 bytes
constexpr int kTileBytes = 256 * kRowBytes;         // 32 KiB per operand tile
constexpr int kStageBytes = 2 * kTileBytes;          // A + W
constexpr int kStages = 2;
constexpr int kGroupM = 16;          // tile rows per group of the walk

// Zero source for pieces past K (global loads must come from somewhere).
__device__ __attribute__((aligned(256))) uint32_t g_lpn_zero[64];

__device__ __forceinline__ void wait_vm(int n) {
  // s_waitcnt vmcnt(n) with expcnt / lgkmcnt at their maxima; n is 0 or 16.
  if (n == 0)
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8) | (0 << 14));
  else
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8) | (1 << 14));  // vmcnt = 16
}

__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Per-lane part of a chunk load: lane l of an instruction covers tile row
// 8*inst + (l >> 3) and the 16-byte piece (l & 7) ^ ((row >> 1) & 7).  Since
// (row >> 1) & 7 = ((inst & 1) * 4 + (l >> 4)) & 7, the piece depends only on
// the lane and the parity of the instruction.
struct LoadLane {
  int rsub;        // row within the instruction's 8 rows
  int piece[2];    // piece for even / odd instructions
};

__device__ __forceinline__ LoadLane load_lane(int lane) {
  LoadLane L;
  L.rsub = lane >> 3;
  const int slot = lane & 7;
  L.piece[0] = slot ^ ((lane >> 4) & 7);
  L.piece[1] = slot ^ ((4 + (lane >> 4)) & 7);
  return L;
}

// Issue the 16 direct-to-LDS loads of this wave for one chunk: 8 of A's 32
// instructions and 8 of W's.  Rows past M (N) read the last row; pieces past
// K read the zero block.
__device__ __forceinline__ void issue(char *stage, int wave, const LoadLane &L,
                                      const uint16_t *__restrict__ A,
                                      const uint16_t *__restrict__ W, int m0, int n0, int M,
                                      int N, int K, int k0) {
  const uint16_t *zero = reinterpret_cast<const uint16_t *>(g_lpn_zero);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int inst = wave * 8 + j;  // 0..31, wave-uniform
    const int r = inst * 8 + L.rsub;
    const int k = k0 + L.piece[j & 1] * 8;
    const uint16_t *pa = A + ((size_t)(unsigned)min(m0 + r, M - 1) * (unsigned)K + (unsigned)k);
    const uint16_t *pw = W + ((size_t)(unsigned)min(n0 + r, N - 1) * (unsigned)K + (unsigned)k);
    __builtin_amdgcn_global_load_lds(k < K ? pa : zero, (lds_void_t *)(stage + inst * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(k < K ? pw : zero, (lds_void_t *)(stage + kTileBytes + inst * 1024), 16, 0, 0);
  }
}

__global__ __launch_bounds__(256, 1) void lazy_prenorm_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W, uint16_t *__restrict__ Cout,
    float *__restrict__ rstd_out, int M, int N, int K, float inv_k, float eps, int tiles_m,
    int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageBytes];
  __shared__ float rs_lds[kTM];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;

  // Tile of this workgroup: each XCD (workgroups are dealt to the 8 XCDs in
  // turn) walks a contiguous run of the grouped order.
  const int T = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int q = T >> 3, rr8 = T & 7, x = bid & 7;
  const int lin = x * q + min(x, rr8) + (bid >> 3);
  const int group = lin / (kGroupM * tiles_n);
  const int gm0 = group * kGroupM;
  const int gsz = min(kGroupM, tiles_m - gm0);
  const int within = lin - group * kGroupM * tiles_n;
  const int tm = gm0 + within % gsz;
  const int tn = within / gsz;
  const int m0 = tm * kTM, n0 = tn * kTN;

  f32x4 acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float sumsq = 0.f;  // thread t: row t of the tile

  const int nchunks = (K + kKC - 1) / kKC;
  const LoadLane L = load_lane(lane);
  issue(lds, wave, L, A, W, m0, n0, M, N, K, 0);
  const int swz = (m >> 1) & 7;  // ((row >> 1) & 7) of every row this lane reads
  for (int c = 0; c < nchunks; ++c) {
    // This wave's loads of chunk c have landed and its reads of chunk c-1 have
    // returned; after the barrier the same holds for all waves, so chunk c is
    // complete and the other stage may be refilled.
    wait_vm(0);
    wait_lgkm0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (c + 1 < nchunks)
      issue(lds + ((c + 1) & 1) * kStageBytes, wave, L, A, W, m0, n0, M, N, K, (c + 1) * kKC);
    const char *sa = lds + (c & 1) * kStageBytes;
    const char *sw = sa + kTileBytes;
#pragma unroll
    for (int t = 0; t < kKC / 32; ++t) {
      const int slot = ((4 * t + g) ^ swz) * 16;
      bf16x8 aop[8], wop[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        aop[b] = *reinterpret_cast<const bf16x8 *>(sa + (wm * 128 + b * 16 + m) * kRowBytes + slot);
        wop[b] = *reinterpret_cast<const bf16x8 *>(sw + (wn * 128 + b * 16 + m) * kRowBytes + slot);
      }
#pragma unroll
      for (int rb = 0; rb < 8; ++rb)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop[cb], aop[rb], acc[rb][cb], 0, 0, 0);
    }
    // Row sums of squares on the vector unit: thread t adds the squares of
    // row t of this chunk (its 8 pieces, wherever the swizzle put them).
    {
      const int srow = (tid >> 1) & 7;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(sa + tid * kRowBytes + ((p ^ srow) * 16));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float lo = bf16_lo(v[w]), hi = bf16_hi(v[w]);
          sumsq = fmaf(lo, lo, sumsq);
          sumsq = fmaf(hi, hi, sumsq);
        }
      }
    }
  }

  // rstd of the tile's 256 rows.
  {
    const float r = 1.0f / sqrtf(sumsq * inv_k + eps);
    rs_lds[tid] = r;
    if (tn == 0 && rstd_out != nullptr && m0 + tid < M) rstd_out[m0 + tid] = r;
  }
  __syncthreads();

  // Epilogue: block (rb, cb) of C^T: lane (m, g) holds C[row][4g .. 4g+3] of
  // row = m0 + wm*128 + rb*16 + m, columns n0 + wn*128 + cb*16 + 4g ...
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    const int lr = wm * 128 + rb * 16 + m;
    const int row = m0 + lr;
    const float s = rs_lds[lr];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int col = n0 + wn * 128 + cb * 16 + 4 * g;
      const f32x4 v = acc[rb][cb];
      const u32x2 o = {pack_bf16x2(v[0] * s, v[1] * s), pack_bf16x2(v[2] * s, v[3] * s)};
      if (row < M && col < N) *reinterpret_cast<u32x2 *>(Cout + (size_t)row * N + col) = o;
    }
  }
}

}  // namespace

hipError_t launch_lazy_prenorm_gemm(int64_t M, int64_t N, int64_t K, const void *A, const void *W,
                                    float eps, void *C, float *rstd, hipStream_t st) {
  const int tiles_m = (int)((M + kTM - 1) / kTM), tiles_n = (int)((N + kTN - 1) / kTN);
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  lazy_prenorm_gemm_kernel<<<dim3((uint32_t)tiles), 256, 0, st>>>(
      static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(W), static_cast<uint16_t *>(C),
      rstd, (int)M, (int)N, (int)K, (float)(1.0 / (double)K), eps, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace mhc
