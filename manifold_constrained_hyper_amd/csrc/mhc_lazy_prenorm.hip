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
// gfx950 design (the page's kernel is written for another GPU; this one is
// laid out for CDNA4):
//  * workgroup tile 256 x 256 of C, 8 waves (two per SIMD, so one wave's LDS
//    reads and barrier waits hide behind the other's matrix work); each wave
//    owns 128 A rows x 64 W rows as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16
//    (128 accumulator registers);
//  * A and W move to LDS in 64-wide k-chunks by direct-to-LDS loads
//    (global_load_lds_dwordx4: one instruction fills 8 rows of 128 bytes),
//    two stages of 64 KiB; the loads are issued from inline asm with an
//    SGPR tile base and per-lane 32-bit row offsets, and waited for with an
//    explicit vmcnt before the chunk's barrier (the compiler would otherwise
//    wait for every outstanding LDS DMA before each LDS read);
//  * within a 128-byte row the 16-byte pieces are XOR-swizzled by
//    ((row >> 1) & 7), so 16 consecutive rows read at one piece index hit 16
//    distinct bank groups (LDS serves 256 bytes per clock);
//  * operands of k-step t+1 are read while the MFMAs of step t run (two
//    register sets of 24 VGPRs), one LDS read after each MFMA (scheduling
//    group barriers keep the compiler from sinking the reads next to their
//    use);
//  * each block computes C^T = W A^T (W as the MFMA A operand), so a lane
//    ends with runs of 4 consecutive output columns of one row: the epilogue
//    scales them by that row's rstd, pairs runs across the two lane halves
//    (v_permlane32_swap) and stores 16 bytes;
//  * the row sums of squares run on the vector unit beside the matrix core:
//    thread t adds the squares of half of row t >> 1 of every A chunk (four
//    independent partial sums, one v_dot2_f32_bf16 per packed pair);
//  * tiles are walked in groups of 4 tile rows, each XCD taking a contiguous
//    run of the order.
#include "mhc_device.h"
#include "mhc_launch.h"

#include <algorithm>

namespace mhc {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;             // workgroup tile (rows of A and of W)
constexpr int kKC = 64;                // k per chunk
constexpr int kRB = kKC * 2;           // 128 bytes per tile row per chunk
constexpr int kPieces = kKC / 8;       // 16-byte pieces per row
constexpr int kTileBytes = kTile * kRB;
constexpr int kStageBytes = 2 * kTileBytes;  // A tile + W tile
constexpr int kStages = 2;
constexpr int kRowsPerInst = 1024 / kRB;                // 8 rows per DMA instruction
constexpr int kWaves = 8;
constexpr int kInstPerWave = kTile / kRowsPerInst / kWaves;  // 4 per operand
constexpr int kLoadsPerWave = 2 * kInstPerWave;         // vmcnt per chunk
constexpr int kSteps = kKC / 16;                        // MFMA k-steps per chunk
constexpr int kGroupM = 4;

// Zero source for pieces past K (global loads must come from somewhere).
__device__ __attribute__((aligned(256))) uint32_t g_lpn_zero[64];

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Direct-to-LDS 16-byte loads: lane i's data lands at M0 + 16 i.
__device__ __forceinline__ void dma_saddr(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory");
}
__device__ __forceinline__ void dma_vaddr(const void *vaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(vaddr), "s"(lds_addr) : "memory");
}
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }
// Workgroup barrier for LDS only: this wave's LDS accesses have completed;
// outstanding global loads (the next tile's chunks) are not waited for.
__device__ __forceinline__ void lds_barrier() {
  wait_lgkm0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// lo^2 + hi^2 + acc of a packed bf16 pair in one instruction (bf16 squares
// are exact in fp32).  Written as inline asm: through the builtin, hipcc
// passed element 0 of a 4-word vector for every element.
__device__ __forceinline__ float dot2_sq_bf16(uint32_t v, float acc) {
  asm("v_dot2_f32_bf16 %0, %1, %1, %0" : "+v"(acc) : "v"(v));
  return acc;
}

struct Operands {
  bf16x8 a[4], w[2];
};

__global__ __launch_bounds__(512, 1) void lazy_prenorm_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W, uint16_t *__restrict__ Cout,
    float *__restrict__ rstd_out, int M, int N, int K, float inv_k, float eps, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStageBytes];
  __shared__ float rs_lds[kTile];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j32 = lane & 31, g = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;  // 2 x 4 waves

  // Tiles of this workgroup.  The grouped order (kGroupM tile rows at a time)
  // is cut into 8 contiguous runs, one per XCD (workgroups are dealt to the
  // XCDs in turn); the P workgroups of an XCD walk its run together, taking
  // tiles j, j + P, j + 2 P, ... of it.
  const int T = tiles_m * tiles_n;
  const int G = gridDim.x, bid = blockIdx.x;
  const int x = bid & 7, jw = bid >> 3;
  const int run0 = x * (T >> 3) + min(x, T & 7), runlen = (T >> 3) + (x < (T & 7) ? 1 : 0);
  const int P = (G >> 3) + (x < (G & 7) ? 1 : 0);
  const int ntiles = jw < runlen ? (runlen - 1 - jw) / P + 1 : 0;
  auto tile_of = [&](int it, int &tm, int &tn) {
    const int lin = run0 + jw + it * P;
    const int group = lin / (kGroupM * tiles_n);
    const int gm0 = group * kGroupM;
    const int gsz = min(kGroupM, tiles_m - gm0);
    const int within = lin - group * kGroupM * tiles_n;
    tm = gm0 + within % gsz;
    tn = within / gsz;
  };

  // DMA: this wave issues instructions kInstPerWave*wave + jj of each operand;
  // instruction i fills tile rows 8 i .. 8 i + 7, lane l row 8 i + (l >> 3),
  // slot l & 7, which holds piece slot ^ swz(row).  Rows past M (N) repeat the
  // last row (their outputs are not stored).  The chunks of all the
  // workgroup's tiles form one stream: the first chunks of the next tile are
  // loaded while the current tile's last chunks and its epilogue run.
  const uint32_t rowK2 = (uint32_t)K * 2u;
  const int rsub = lane / kPieces, slot = lane % kPieces;
  uint32_t voa[kInstPerWave], vow[kInstPerWave];
  int pce[kInstPerWave];
  const char *Ab = nullptr, *Wb = nullptr;
  auto dma_tile = [&](int it) {  // point the DMA at tile it
    int tm, tn;
    tile_of(it, tm, tn);
    const int m0 = tm * kTile, n0 = tn * kTile;
#pragma unroll
    for (int jj = 0; jj < kInstPerWave; ++jj) {
      const int r = kRowsPerInst * (kInstPerWave * wave + jj) + rsub;
      pce[jj] = slot ^ swz(r);
      voa[jj] = (uint32_t)(min(m0 + r, M - 1) - m0) * rowK2 + pce[jj] * 16;
      vow[jj] = (uint32_t)(min(n0 + r, N - 1) - n0) * rowK2 + pce[jj] * 16;
    }
    Ab = reinterpret_cast<const char *>(A) + (size_t)m0 * rowK2;
    Wb = reinterpret_cast<const char *>(W) + (size_t)n0 * rowK2;
  };
  auto issue = [&](int stage, int k0) {
    const uint32_t sb = lds_base + stage * kStageBytes + kInstPerWave * wave * 1024;
    const char *ab = Ab + (size_t)k0 * 2, *wb = Wb + (size_t)k0 * 2;
    if (k0 + kKC <= K) {
#pragma unroll
      for (int jj = 0; jj < kInstPerWave; ++jj) {
        dma_saddr(ab, voa[jj], sb + jj * 1024);
        dma_saddr(wb, vow[jj], sb + kTileBytes + jj * 1024);
      }
    } else {  // ragged last chunk: pieces past K read the zero block
      const char *zero = reinterpret_cast<const char *>(g_lpn_zero);
#pragma unroll
      for (int jj = 0; jj < kInstPerWave; ++jj) {
        const bool in = k0 + pce[jj] * 8 < K;
        dma_vaddr(in ? ab + voa[jj] : zero, sb + jj * 1024);
        dma_vaddr(in ? wb + vow[jj] : zero, sb + kTileBytes + jj * 1024);
      }
    }
  };
  const int nchunks = (K + kKC - 1) / kKC;
  const int total = ntiles * nchunks;  // chunks in this workgroup's stream
  int dit = 0, dc = 0;                  // tile and chunk the next DMA fills
  auto issue_next = [&](int stage) {
    if (dc == nchunks) {
      dc = 0;
      dma_tile(++dit);
    }
    issue(stage, dc * kKC);
    ++dc;
  };

  // Operand reads: k-step t of a chunk uses piece 2t + g of row j32 of each
  // 32-row block (the 32x32x16 operand layout: lane l supplies k 8 (l >> 5)
  // .. +7 of row l & 31).
  const int sw = swz(j32);
  const int offa = (wm * 128 + j32) * kRB, offw = kTileBytes + (wn * 64 + j32) * kRB;
  auto read_ops = [&](Operands &o, int stage, int t) {
    const char *st = lds + stage * kStageBytes;
    const int sl = ((2 * t + g) ^ sw) * 16;
#pragma unroll
    for (int b = 0; b < 4; ++b) o.a[b] = *reinterpret_cast<const bf16x8 *>(st + offa + b * 32 * kRB + sl);
#pragma unroll
    for (int b = 0; b < 2; ++b) o.w[b] = *reinterpret_cast<const bf16x8 *>(st + offw + b * 32 * kRB + sl);
  };

  // Row sums of squares: thread t takes row t >> 1, pieces 4 (t & 1) .. +3.
  const int srow = tid >> 1, sh = tid & 1;
  u32x4 sq[kPieces / 2];
  auto read_sq = [&](int stage) {
    const char *st = lds + stage * kStageBytes + srow * kRB;
#pragma unroll
    for (int p = 0; p < kPieces / 2; ++p)
      sq[p] = *reinterpret_cast<const u32x4 *>(st + ((((kPieces / 2) * sh + p) ^ swz(srow)) * 16));
    __builtin_amdgcn_sched_barrier(0);
  };
  float ssp[4] = {0.f, 0.f, 0.f, 0.f};
  auto add_sq = [&]() {
#pragma unroll
    for (int p = 0; p < kPieces / 2; ++p)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        ssp[w] = dot2_sq_bf16(sq[p][w], ssp[w]);
      }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
  auto mfma = [&](const Operands &o) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w[cb], o.a[rb], acc[rb][cb], 0, 0, 0);
    // one LDS read of the next k-step after each of the first six MFMAs
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  if (total == 0) return;  // more workgroups than tiles (uniform per workgroup)
  dma_tile(0);
#pragma unroll
  for (int s = 0; s < kStages; ++s)
    if (s < total) issue_next(s);
  if (total >= kStages) wait_vm<(kStages - 1) * kLoadsPerWave>();
  else wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  Operands o0, o1;
  read_ops(o0, 0, 0);
  read_sq(0);

  int gc = 0;  // position in the chunk stream
  for (int it = 0; it < ntiles; ++it) {
    for (int c = 0; c < nchunks; ++c, ++gc) {
      const int st = gc % kStages;
      // k-steps 0 .. kSteps-2 of this chunk, each reading the next step's operands
#pragma unroll
      for (int t = 0; t + 1 < kSteps; t += 2) {
        read_ops(o1, st, t + 1);
        mfma(o0);
        if (t == 0) add_sq();
        if (t + 2 < kSteps) {
          read_ops(o0, st, t + 2);
          mfma(o1);
        }
      }
      // Chunk gc+1 of the stream has landed (this wave's loads, then the
      // barrier for all waves) and every read of chunk gc has returned, so
      // its stage may be refilled with chunk gc + kStages.
      if (gc + kStages - 1 < total) wait_vm<(kStages - 2) * kLoadsPerWave>();
      else wait_vm<0>();
      lds_barrier();
      if (gc + kStages < total) issue_next(st);
      // last k-step; read step 0 of the next chunk (past the stream's end:
      // stale, unused)
      const int sn = (gc + 1) % kStages;
      read_ops(o0, sn, 0);
      read_sq(sn);
      mfma(o1);
    }

    int tm, tn;
    tile_of(it, tm, tn);
    const int m0 = tm * kTile, n0 = tn * kTile;
    float ss = (ssp[0] + ssp[1]) + (ssp[2] + ssp[3]);
    ss += __shfl_xor(ss, 1);
    if (sh == 0) rs_lds[srow] = ss;
    lds_barrier();
    if (tid < kTile) {
      const float r = 1.0f / sqrtf(rs_lds[tid] * inv_k + eps);
      if (tn == 0 && rstd_out != nullptr && m0 + tid < M) rstd_out[m0 + tid] = r;
      rs_lds[tid] = r;  // each thread reads and rewrites only its own row
    }
    lds_barrier();

    // Epilogue: block (rb, cb) of C^T: lane holds row j32 of A block rb and
    // columns 8 q + 4 g .. +3 (q = 0..3) of W block cb.  For each pair of
    // column groups (q, q + 1) one v_permlane32_swap per word gives lane g
    // all 8 columns of group q + g (16 bytes): lanes 0-31 trade their group
    // q + 1 half for lanes 32-63's group q half.  rs_lds is next written
    // after the next tile's first chunk barrier.
    const bool interior = (m0 + kTile <= M) && (n0 + kTile <= N);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int lr = wm * 128 + rb * 32 + j32;
      const int row = m0 + lr;
      const float sc = rs_lds[lr];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const f32x16 v = acc[rb][cb];
#pragma unroll
        for (int qp = 0; qp < 4; qp += 2) {
          const uint32_t a0 = pack_bf16x2(v[4 * qp] * sc, v[4 * qp + 1] * sc);
          const uint32_t a1 = pack_bf16x2(v[4 * qp + 2] * sc, v[4 * qp + 3] * sc);
          const uint32_t b0 = pack_bf16x2(v[4 * qp + 4] * sc, v[4 * qp + 5] * sc);
          const uint32_t b1 = pack_bf16x2(v[4 * qp + 6] * sc, v[4 * qp + 7] * sc);
          const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
          const u32x4 ov = {s0[0], s1[0], s0[1], s1[1]};
          const int col = n0 + wn * 64 + cb * 32 + 8 * (qp + g);  // N % 8 == 0: all 8 in range or none
          if (interior || (row < M && col < N)) *reinterpret_cast<u32x4 *>(Cout + (size_t)row * N + col) = ov;
        }
        acc[rb][cb] = f32x16{};
      }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) ssp[w] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Four-wave variant: the same 256 x 256 tiles and direct-to-LDS staging, but
// one wave per SIMD, each owning 128 A rows x 128 W rows as 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (256 accumulator registers, held in the AGPR half
// of the 512-register file a lone wave gets).  Per 16-k step a wave reads
// 4 + 4 operand vectors for 16 MFMAs: two thirds of the eight-wave layout's
// LDS bytes per flop.
//
// With one wave per SIMD nothing hides a stall, so (measured on MI355X):
//  * k moves in 32-wide chunks through four 32 KiB stages, three chunks
//    ahead of the math (with two 64-wide stages, one chunk ahead, waiting
//    for the DMA cost a third of the rate);
//  * every instruction between two MFMAs delays the next one (a register-
//    only loop of 32x32x16 MFMAs reaches 2.13 PFLOP/s from one wave per SIMD,
//    16x16x32 ones only 1.48), so each step's MFMAs are issued in a fixed
//    order with the other work placed between them, and the row sums of
//    squares (v_dot2 on the A operands already in registers, no extra LDS
//    reads) are split between the two waves that hold the same A rows.
constexpr int kWaves4 = 4;
constexpr int kKC4 = 32;                                   // k per chunk
constexpr int kRB4 = kKC4 * 2;                             // 64 bytes per tile row per chunk
constexpr int kTileBytes4 = kTile * kRB4;                  // 16 KiB
constexpr int kStageBytes4 = 2 * kTileBytes4;              // A tile + W tile
constexpr int kStages4 = 4;
constexpr int kRowsPerInst4 = 1024 / kRB4;                 // 16 rows per DMA instruction
constexpr int kInstPerWave4 = kTile / kRowsPerInst4 / kWaves4;  // 4 per operand
constexpr int kLoadsPerWave4 = 2 * kInstPerWave4;          // vmcnt per chunk

// 64-byte rows hold 4 pieces; piece p of row r sits in slot p ^ ((r >> 2) & 3),
// so 16 consecutive rows read at one piece index cover all 64 banks once.
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

struct Operands4 {
  bf16x8 a[4], w[4];
};

__global__ __launch_bounds__(256, 1) void lazy_prenorm_gemm4_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W, uint16_t *__restrict__ Cout,
    float *__restrict__ rstd_out, int M, int N, int K, float inv_k, float eps, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char lds[kStages4 * kStageBytes4];
  __shared__ float rs_lds[kTile];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j32 = lane & 31, g = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;  // 2 x 2 waves

  // Tile walk: as the eight-wave kernel (grouped order, one run per XCD).
  const int T = tiles_m * tiles_n;
  const int G = gridDim.x, bid = blockIdx.x;
  const int x = bid & 7, jw = bid >> 3;
  const int run0 = x * (T >> 3) + min(x, T & 7), runlen = (T >> 3) + (x < (T & 7) ? 1 : 0);
  const int P = (G >> 3) + (x < (G & 7) ? 1 : 0);
  const int ntiles = jw < runlen ? (runlen - 1 - jw) / P + 1 : 0;
  auto tile_of = [&](int it, int &tm, int &tn) {
    const int lin = run0 + jw + it * P;
    const int group = lin / (kGroupM * tiles_n);
    const int gm0 = group * kGroupM;
    const int gsz = min(kGroupM, tiles_m - gm0);
    const int within = lin - group * kGroupM * tiles_n;
    tm = gm0 + within % gsz;
    tn = within / gsz;
  };

  // DMA: wave w issues instructions 4 w .. 4 w + 3 of each operand; one
  // instruction fills 16 rows of 64 bytes, lane l row 16 i + (l >> 2), slot
  // l & 3 (piece slot ^ swz4(row)).  Rows past M (N) repeat the last row.
  const uint32_t rowK2 = (uint32_t)K * 2u;
  const int rsub = lane >> 2, slot = lane & 3;
  const char *Ab = nullptr, *Wb = nullptr;
  int dm0 = 0, dn0 = 0;
  auto dma_tile = [&](int it) {
    int tm, tn;
    tile_of(it, tm, tn);
    dm0 = tm * kTile;
    dn0 = tn * kTile;
    Ab = reinterpret_cast<const char *>(A) + (size_t)dm0 * rowK2;
    Wb = reinterpret_cast<const char *>(W) + (size_t)dn0 * rowK2;
  };
  auto issue = [&](int stage, int k0) {
    const uint32_t sb = lds_base + stage * kStageBytes4 + kInstPerWave4 * wave * 1024;
    const char *ab = Ab + (size_t)k0 * 2, *wb = Wb + (size_t)k0 * 2;
    auto off = [&](int jj, int base0, int lim, int &pc) {
      const int r = kRowsPerInst4 * (kInstPerWave4 * wave + jj) + rsub;
      pc = slot ^ swz4(r);
      return (uint32_t)(min(base0 + r, lim - 1) - base0) * rowK2 + pc * 16;
    };
    if (k0 + kKC4 <= K) {
#pragma unroll
      for (int jj = 0; jj < kInstPerWave4; ++jj) {
        int pc;
        dma_saddr(ab, off(jj, dm0, M, pc), sb + jj * 1024);
        dma_saddr(wb, off(jj, dn0, N, pc), sb + kTileBytes4 + jj * 1024);
      }
    } else {  // ragged last chunk: pieces past K read the zero block
      const char *zero = reinterpret_cast<const char *>(g_lpn_zero);
#pragma unroll
      for (int jj = 0; jj < kInstPerWave4; ++jj) {
        int pc;
        const uint32_t oa = off(jj, dm0, M, pc), ow = off(jj, dn0, N, pc);
        const bool in = k0 + pc * 8 < K;
        dma_vaddr(in ? ab + oa : zero, sb + jj * 1024);
        dma_vaddr(in ? wb + ow : zero, sb + kTileBytes4 + jj * 1024);
      }
    }
  };
  const int nchunks = (K + kKC4 - 1) / kKC4;
  const int total = ntiles * nchunks;
  int dit = 0, dc = 0;
  auto issue_next = [&](int stage) {
    if (dc == nchunks) {
      dc = 0;
      dma_tile(++dit);
    }
    issue(stage, dc * kKC4);
    ++dc;
  };

  // Operand read r (0..3: a[r], 4..7: w[r-4]) of 16-k step t (0, 1) of a
  // chunk: piece 2t + g of row j32 of each 32-row block (the 32x32x16 operand
  // layout: lane l supplies k 8 (l >> 5) .. +7 of row l & 31).  The waves
  // with wn = 1 hold their A blocks rotated by two (a[r] is block
  // (r + 2 wn) & 3), so the blocks whose squares a wave sums are a[0] and
  // a[1] in every wave: no selection in the MFMA stream.
  const int sw = swz4(j32);
  const int offw = kTileBytes4 + (wn * 128 + j32) * kRB4;
  int offa[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) offa[r] = (wm * 128 + ((r + 2 * wn) & 3) * 32 + j32) * kRB4;
  auto read_one = [&](Operands4 &o, int stage, int t, int r) {
    const char *st = lds + stage * kStageBytes4;
    const int sl = ((2 * t + g) ^ sw) * 16;
    if (r < 4) o.a[r] = *reinterpret_cast<const bf16x8 *>(st + offa[r] + sl);
    else o.w[r - 4] = *reinterpret_cast<const bf16x8 *>(st + offw + (r - 4) * 32 * kRB4 + sl);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};
  // Sums of squares: each wave sums a[0] and a[1], i.e. A blocks 2 wn and
  // 2 wn + 1 of its 128 rows (lane: row j32 of the block, k-half g).
  float ssq[2] = {0.f, 0.f};
  auto sq_slot = [&](const Operands4 &o, int i) {
    if (i >= 8 && i < 12) {
      const int b = (i - 8) >> 1, h = (i - 8) & 1;  // a[b], words 2 h, 2 h + 1
      const u32x4 v = __builtin_bit_cast(u32x4, o.a[b]);
      ssq[b] = dot2_sq_bf16(v[2 * h], ssq[b]);
      ssq[b] = dot2_sq_bf16(v[2 * h + 1], ssq[b]);
    }
  };
  // One 16-k step: its 16 MFMAs in a fixed order, `slot(i)` placing other
  // work after MFMA i; scheduling barriers keep that order.
  auto step = [&](const Operands4 &o, auto &&slotf) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rb = i >> 2, cb = i & 3;
      acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.w[cb], o.a[rb], acc[rb][cb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      slotf(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (total == 0) return;
  dma_tile(0);
#pragma unroll
  for (int s = 0; s < kStages4; ++s)
    if (s < total) issue_next(s);
  // chunk 0 has landed for this wave, then for every wave
  if (total >= 4) wait_vm<3 * kLoadsPerWave4>();
  else if (total == 3) wait_vm<2 * kLoadsPerWave4>();
  else if (total == 2) wait_vm<kLoadsPerWave4>();
  else wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  Operands4 o0, o1;
#pragma unroll
  for (int r = 0; r < 8; ++r) read_one(o0, 0, 0, r);

  int gc = 0;
  for (int it = 0; it < ntiles; ++it) {
    for (int c = 0; c < nchunks; ++c, ++gc) {
      const int st = gc % kStages4;
      // step 0: the reads of step 1 after MFMAs 0-7
      step(o0, [&](int i) {
        if (i < 8) read_one(o1, st, 1, i);
        sq_slot(o0, i);
      });
      // step 1: after its first MFMA, wait until chunk gc+1 has landed and
      // this wave's reads of chunk gc have returned, then the barrier: every
      // wave is past chunk gc, so its stage takes chunk gc + 4.  The reads of
      // chunk gc+1's first step follow MFMAs 8-15.
      const int ahead = total - 1 - gc;  // chunks after this one
      step(o1, [&](int i) {
        if (i == 0) {
          if (ahead >= 3) wait_vm<2 * kLoadsPerWave4>();
          else if (ahead == 2) wait_vm<kLoadsPerWave4>();
          else wait_vm<0>();
          lds_barrier();
          if (gc + kStages4 < total) issue_next(st);
        }
        if (i >= 8) read_one(o0, (gc + 1) % kStages4, 0, i - 8);  // past the stream's end: stale, unused
        sq_slot(o1, i);
      });
    }

    int tm, tn;
    tile_of(it, tm, tn);
    const int m0 = tm * kTile, n0 = tn * kTile;
    // Row sums: the two k-halves of a row live in lanes j32 and j32 + 32.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float ss = ssq[b] + __shfl_xor(ssq[b], 32);
      if (g == 0) rs_lds[wm * 128 + (2 * wn + b) * 32 + j32] = ss;
      ssq[b] = 0.f;
    }
    lds_barrier();
    if (tid < kTile) {
      const float r = 1.0f / sqrtf(rs_lds[tid] * inv_k + eps);
      if (tn == 0 && rstd_out != nullptr && m0 + tid < M) rstd_out[m0 + tid] = r;
      rs_lds[tid] = r;
    }
    lds_barrier();

    // Epilogue: block (rb, cb) of C^T; lane holds row j32 of A block rb and
    // columns 8 q + 4 g .. +3 of W block cb; runs paired across lane halves
    // by v_permlane32_swap, 16 bytes per lane.
    const bool interior = (m0 + kTile <= M) && (n0 + kTile <= N);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int lr = wm * 128 + ((rb + 2 * wn) & 3) * 32 + j32;  // acc[rb] holds A block (rb + 2 wn) & 3
      const int row = m0 + lr;
      const float sc = rs_lds[lr];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const f32x16 v = acc[rb][cb];
#pragma unroll
        for (int qp = 0; qp < 4; qp += 2) {
          const uint32_t a0 = pack_bf16x2(v[4 * qp] * sc, v[4 * qp + 1] * sc);
          const uint32_t a1 = pack_bf16x2(v[4 * qp + 2] * sc, v[4 * qp + 3] * sc);
          const uint32_t b0 = pack_bf16x2(v[4 * qp + 4] * sc, v[4 * qp + 5] * sc);
          const uint32_t b1 = pack_bf16x2(v[4 * qp + 6] * sc, v[4 * qp + 7] * sc);
          const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
          const u32x4 ov = {s0[0], s1[0], s0[1], s1[1]};
          const int col = n0 + wn * 128 + cb * 32 + 8 * (qp + g);
          if (interior || (row < M && col < N)) *reinterpret_cast<u32x4 *>(Cout + (size_t)row * N + col) = ov;
        }
        acc[rb][cb] = f32x16{};
      }
    }
  }
}

}  // namespace

hipError_t launch_lazy_prenorm_gemm(int64_t M, int64_t N, int64_t K, const void *A, const void *W,
                                    float eps, void *C, float *rstd, hipStream_t st) {
  const int tiles_m = (int)((M + kTile - 1) / kTile), tiles_n = (int)((N + kTile - 1) / kTile);
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  // persistent: one workgroup per compute unit (the LDS stages allow one);
  // at least 8, so that each XCD run of the tile order has a workgroup
  const int64_t grid = std::min<int64_t>(tiles, std::max(device_cus(), 8));
  if (tune(kTuneLpnAlgo) == 1)
    lazy_prenorm_gemm4_kernel<<<dim3((uint32_t)grid), kWaves4 * 64, 0, st>>>(
        static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(W), static_cast<uint16_t *>(C),
        rstd, (int)M, (int)N, (int)K, (float)(1.0 / (double)K), eps, tiles_m, tiles_n);
  else
    lazy_prenorm_gemm_kernel<<<dim3((uint32_t)grid), kWaves * 64, 0, st>>>(
        static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(W), static_cast<uint16_t *>(C),
        rstd, (int)M, (int)N, (int)K, (float)(1.0 / (double)K), eps, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace mhc
