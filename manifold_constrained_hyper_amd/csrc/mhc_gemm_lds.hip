// Fused coefficient product and sum of squares with X staged through LDS.
//
// Same arithmetic as gemm_rms_kernel (mhc_gemm_rms.hip): per row tile and
// K-slice, the partial logits X_t . phi ([mHC-cutile] = page "mHC 算法分析 &
// cutile 高效实现", sections 2.1, 3.1, 5.1) and the partial sum of X_t^2
// (section 2.2) are written as fp32 [S, B, N+1] for the combine kernel.
//
// What changes is how X reaches the matrix cores.  The MFMA A operand wants
// 16 rows x 16 bytes per instruction, and reading HBM in that shape (16 rows x
// 64 bytes per load instruction) leaves a good part of the bandwidth unused.
// Here X is read row-contiguously instead, by the gfx950 direct-to-LDS load
// (global_load_lds_dwordx4: each lane's 16 bytes land at LDS base + 16*lane),
// into a ring of STAGES chunk buffers, and the A operands are read back from
// LDS.  So that those reads are free of bank conflicts, the 16-byte pieces of
// row r are stored XOR-swizzled (piece p at slot p ^ (r & 15)); the swizzle is
// applied through the per-lane source addresses, so every load instruction
// still covers whole contiguous row segments.
//
// phi is consumed in a packed copy, written by pack_phi_kernel (mhc_pack.hip)
// into the workspace at the start of every call: for each 32-k step and 16-column
// block, the 64 lanes' B operands (8 consecutive k of one column) are one
// contiguous KiB, so phi also moves by direct-to-LDS loads, one instruction
// per KiB, with no transposition on the critical path.  Columns past N and k
// past K are zero in the packed copy.  X pieces past K are read from a zeroed
// 256-byte block of the workspace instead of past the end of the row.
//
// fp32 phi (the *_phi32 calls): pack_phi32_kernel splits each value into
// phi_hi = bf16(phi) and phi_lo = bf16(phi - phi_hi) (together within 2^-16
// of phi, relative) and writes, per 32-k step, the NB hi blocks followed by
// the NB lo blocks; the product then runs two MFMAs per block,
// X.phi_hi + X.phi_lo, into the same fp32 accumulator (bf16 X times either
// part is exact in fp32).
//
// Pipeline per workgroup (W waves, 16*MB*W rows): the loads of chunks
// c+1 .. c+STAGES-1 are in flight while chunk c is multiplied.  Each wave
// waits only for its own share of chunk c (s_waitcnt vmcnt), then one barrier
// makes the whole chunk visible and frees the slot of chunk c-1 for refill.
//
// Eight waves (the E4M3 default) make 128-row tiles, so each chunk's phi
// blocks are staged once per 128 rows instead of 64: at n = 8 the staged
// phi bytes per X byte fall from 2.5 to 1.25 (E4M3), and two waves per SIMD
// overlap one wave's LDS reads with the other's MFMAs.
#include "mhc_device.h"
#include "mhc_launch.h"

#include <type_traits>

namespace mhc {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

template <int NS, int MB, int KC, int STAGES, int XB, int P2 = 1, int W = 4>
struct LdsTile {
  static constexpr int N = NS * NS + 2 * NS;
  static constexpr int NP = N + 1;
  static constexpr int NB = (N + 15) / 16;
  static constexpr int PB = NB * P2;                 // packed phi blocks per 32-k step
  static constexpr int RT = 16 * MB * W;             // rows per workgroup
  static constexpr int T = KC / 32;                  // MFMA k-steps per chunk
  static constexpr int EPP = 16 / XB;                // X elements per 16-byte piece
  static constexpr int ROW_BYTES = KC * XB;          // one row of a chunk in LDS
  static constexpr int PIECES = KC / EPP;            // 16-byte pieces per row per chunk
  static constexpr int RPI = 64 / PIECES;            // rows per load instruction
  static constexpr int XI = RT * PIECES / 64;        // X load instructions per chunk
  static constexpr int PI = T * PB;                  // phi load instructions per chunk
  static constexpr int XI_W = XI / W;                // X loads per wave
  // phi load j*W + w is wave w's j-th: waves below PI_REM issue PI_HI, the
  // others PI_LO (equal when W divides PI).
  static constexpr int PI_LO = PI / W, PI_REM = PI % W, PI_HI = PI_LO + (PI_REM ? 1 : 0);
  static constexpr int VM_HI = XI_W + PI_HI, VM_LO = XI_W + PI_LO;  // loads per chunk per wave
  static constexpr int X_BYTES = RT * ROW_BYTES;
  static constexpr int P_BYTES = PI * 1024;
  static constexpr int STAGE_BYTES = X_BYTES + P_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(W == 4 || W == 8, "four or eight waves");
  static_assert(PIECES >= 16 && PIECES <= 64, "swizzle needs 16..64 pieces per row");
  static_assert(XI % W == 0, "X load instructions must split evenly over the waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2 && STAGES <= 6, "pipeline depth");
  static_assert((STAGES - 2) * VM_HI < 64, "vmcnt range");
};

// s_waitcnt with only the vector-memory counter constrained (expcnt and
// lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int NS, int MB, int KC, int STAGES, int XB, int P2, int W>
__device__ __forceinline__ void issue_chunk(char *lds, int slot, int wave, int lane,
                                           const uint8_t *__restrict__ X,
                                           const uint16_t *__restrict__ phip,
                                           const uint16_t *__restrict__ zero, int row0, int B,
                                           int K, int k0) {
  using L = LdsTile<NS, MB, KC, STAGES, XB, P2, W>;
  char *xs = lds + slot * L::STAGE_BYTES;
  char *ps = xs + L::X_BYTES;
  const int slot_in_row = lane % L::PIECES;
#pragma unroll
  for (int j = 0; j < L::XI_W; ++j) {
    const int inst = wave * L::XI_W + j;
    const int rr = inst * L::RPI + lane / L::PIECES;          // row within the tile
    const int piece = slot_in_row ^ (rr & 15);
    const int k = k0 + piece * L::EPP;
    const int row = min(row0 + rr, B - 1);
    const void *src = (k < K) ? static_cast<const void *>(X + ((size_t)row * K + k) * XB)
                              : static_cast<const void *>(zero);
    __builtin_amdgcn_global_load_lds(src, (lds_void *)(xs + inst * 1024), 16, 0, 0);
  }
  const int kstep0 = k0 / 32;
#pragma unroll
  for (int j = 0; j < L::PI_HI; ++j) {
    const int inst = j * W + wave;                             // = t * PB + block
    if (j < L::PI_LO || wave < L::PI_REM) {                    // wave-uniform
      const uint16_t *src = phip + ((size_t)(kstep0 * L::PB + inst) * 64 + lane) * 8;
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(ps + inst * 1024), 16, 0, 0);
    }
  }
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Wait until at most `later` chunks' loads of this wave are outstanding
// (later <= STAGES - 2; V = this wave's loads per chunk).
template <int STAGES, int V>
__device__ __forceinline__ void wait_chunks_v(int later) {
  if (STAGES >= 6 && later >= 4) wait_vmcnt<(STAGES >= 6 ? 4 : 0) * V>();
  else if (STAGES >= 5 && later >= 3) wait_vmcnt<(STAGES >= 5 ? 3 : 0) * V>();
  else if (STAGES >= 4 && later >= 2) wait_vmcnt<(STAGES >= 4 ? 2 : 0) * V>();
  else if (later >= 1) wait_vmcnt<V>();
  else wait_vmcnt<0>();
}

template <int NS, int MB, int KC, int STAGES, int XB, int P2, int W>
__device__ __forceinline__ void wait_chunks(int later, int wave) {
  using L = LdsTile<NS, MB, KC, STAGES, XB, P2, W>;
  if (L::PI_REM == 0 || wave < L::PI_REM) wait_chunks_v<STAGES, L::VM_HI>(later);  // wave-uniform
  else wait_chunks_v<STAGES, L::VM_LO>(later);
}

template <int NS, int MB, int KC, int STAGES, int XB, int P2, int W>
__global__ __launch_bounds__(W * 64) void gemm_rms_lds_kernel(const uint8_t *__restrict__ X,
                                                              const uint16_t *__restrict__ phip,
                                                              const uint16_t *__restrict__ zero,
                                                              float *__restrict__ ws, int B, int K,
                                                              int kslice) {
  using L = LdsTile<NS, MB, KC, STAGES, XB, P2, W>;
  __shared__ __attribute__((aligned(1024))) char lds[L::LDS_BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int s = blockIdx.y;
  const int k_begin = s * kslice;
  const int k_end = min(K, k_begin + kslice);
  const int nchunks = (k_end - k_begin + KC - 1) / KC;
  const int row0 = blockIdx.x * L::RT;

  f32x4 acc[MB][L::NB], gram[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    gram[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < L::NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

#pragma unroll
  for (int c = 0; c < STAGES - 1; ++c)
    if (c < nchunks)
      issue_chunk<NS, MB, KC, STAGES, XB, P2, W>(lds, c, wave, lane, X, phip, zero, row0, B, K,
                                         k_begin + c * KC);

  for (int c = 0; c < nchunks; ++c) {
    // This wave's loads of chunk c have landed and its LDS reads of chunk
    // c-1 have returned; after the barrier the same holds for every wave, so
    // chunk c is complete and the slot of chunk c-1 may be refilled.  (A bare
    // s_barrier: a fenced __syncthreads would also wait for the loads still
    // in flight for the later chunks.)
    wait_chunks<NS, MB, KC, STAGES, XB, P2, W>(min(STAGES - 2, nchunks - 1 - c), wave);
    wait_lgkmcnt0();
    asm volatile("" ::: "memory");  // no memory access moves across the barrier
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int cn = c + STAGES - 1;
    if (cn < nchunks)
      issue_chunk<NS, MB, KC, STAGES, XB, P2, W>(lds, cn % STAGES, wave, lane, X, phip, zero, row0, B,
                                         K, k_begin + cn * KC);
    const char *xs = lds + (c % STAGES) * L::STAGE_BYTES;
    const char *ps = xs + L::X_BYTES;
    // The operands of k-step t+1 are read from LDS while the MFMAs of k-step
    // t run (two register sets, the order pinned by scheduling barriers), so
    // only the first k-step of a chunk waits for a full LDS round trip.  Left
    // to itself the compiler reads two B operands at a time and waits for
    // each pair, three round trips per k-step at n = 8.
    using RawA = std::conditional_t<XB == 2, bf16x8, u32x2>;
    struct Ops {
      bf16x8 b[L::PB];
      RawA a[MB];
    };
    auto read_ops = [&](Ops &o, int t) {
#pragma unroll
      for (int j = 0; j < L::PB; ++j)
        o.b[j] = *reinterpret_cast<const bf16x8 *>(ps + (t * L::PB + j) * 1024 + lane * 16);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int rr = wave * 16 * MB + mb * 16 + m;
        if constexpr (XB == 2) {
          const int slot = (4 * t + g) ^ m;  // rr & 15 == m
          o.a[mb] = *reinterpret_cast<const bf16x8 *>(xs + rr * L::ROW_BYTES + slot * 16);
        } else {
          // E4M3: k = 32t + 8g .. +7 is the (g & 1) half of piece 2t + g/2.
          const int slot = (2 * t + (g >> 1)) ^ m;
          o.a[mb] = *reinterpret_cast<const u32x2 *>(xs + rr * L::ROW_BYTES + slot * 16 + (g & 1) * 8);
        }
      }
    };
    auto mfma_ops = [&](const Ops &o) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        bf16x8 a;
        if constexpr (XB == 2) a = o.a[mb];
        else a = __builtin_bit_cast(bf16x8, fp8x8_to_bf16(o.a[mb]));  // exact widening
#pragma unroll
        for (int nb = 0; nb < L::NB; ++nb) {
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, o.b[nb], acc[mb][nb], 0, 0, 0);
          if constexpr (P2 == 2)  // the low part of an fp32 phi
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, o.b[L::NB + nb], acc[mb][nb], 0, 0, 0);
        }
        gram[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, gram[mb], 0, 0, 0);
      }
    };
    Ops ops[2];
    read_ops(ops[0], 0);
#pragma unroll
    for (int t = 0; t < L::T; ++t) {
      if (t + 1 < L::T) read_ops(ops[(t + 1) & 1], t + 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_ops(ops[t & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // D layout of the 16x16 MFMA: lane (m, g) holds rows 4g..4g+3 of column m.
  float *wsl = ws + (size_t)s * B * L::NP;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rbase = row0 + wave * 16 * MB + mb * 16;
#pragma unroll
    for (int nb = 0; nb < L::NB; ++nb) {
      const int col = nb * 16 + m;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = rbase + 4 * g + v;
        if (row < B && col < L::N) wsl[(size_t)row * L::NP + col] = acc[mb][nb][v];
      }
    }
    if (g == (m >> 2)) {  // Gram diagonal (m, m): lane (m, m/4), element m%4
      const int row = rbase + m;
      if (row < B) wsl[(size_t)row * L::NP + L::N] = gram[mb][m & 3];
    }
  }
}

// The same product with X and phi through registers (bf16 X; the n = 8
// route).  At n = 8 a 256-k chunk of phi is 40 KiB, so an LDS ring cannot
// hold both enough X in flight and 512-byte row pieces (the 128-k chunks of
// gemm_rms_lds_kernel read rows in 256-byte pieces, which HBM serves at about
// 4 TB/s against 6 for 512-byte ones).  Here every wave loads its share of
// chunk c+D (X rows row-contiguously, 1 KiB per instruction; phi blocks of
// the packed copy) into one of D register sets while chunk c is multiplied,
// and writes a set into single LDS slots (X XOR-swizzled as above) just
// before the chunk's barrier.  All waits on those loads are the compiler's
// own (register dependences), so D-1 chunks stay in flight at every point;
// no direct-to-LDS load is used.
template <int NS, int W, int KC>
struct XrTile {
  static constexpr int N = NS * NS + 2 * NS;
  static constexpr int NP = N + 1;
  static constexpr int NB = (N + 15) / 16;
  static constexpr int PB = NB;
  static constexpr int RT = 16 * W;                  // rows per workgroup (one 16-row block per wave)
  static constexpr int T = KC / 32;                  // MFMA k-steps per chunk
  static constexpr int PIECES = KC / 8;              // 16-byte pieces per row per chunk
  static constexpr int RPI = 64 / PIECES;            // rows per load instruction
  static constexpr int XI = RT * PIECES / 64;        // X load instructions per chunk
  static constexpr int XI_W = XI / W;
  static constexpr int PI = T * PB;                  // phi blocks (KiB) per chunk
  static constexpr int PI_HI = (PI + W - 1) / W;     // ... loaded by a wave at most
  static constexpr int ROW_BYTES = KC * 2;
  static constexpr int X_BYTES = RT * ROW_BYTES;
  static constexpr int P_BYTES = PI * 1024;
  static constexpr int LDS_BYTES = X_BYTES + P_BYTES;
  static_assert(PIECES >= 16 && PIECES <= 64, "swizzle needs 16..64 pieces per row");
  static_assert(XI % W == 0, "X load instructions must split evenly over the waves");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int NS, int W, int KC, int D>
__global__ __launch_bounds__(W * 64) void gemm_rms_xreg_kernel(const uint16_t *__restrict__ X,
                                                               const uint16_t *__restrict__ phip,
                                                               const uint16_t *__restrict__ zero,
                                                               float *__restrict__ ws, int B, int K,
                                                               int kslice) {
  using L = XrTile<NS, W, KC>;
  __shared__ __attribute__((aligned(1024))) char lds[L::LDS_BYTES];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int s = blockIdx.y;
  const int k_begin = s * kslice;
  const int k_end = min(K, k_begin + kslice);
  const int nchunks = (k_end - k_begin + KC - 1) / KC;
  const int row0 = blockIdx.x * L::RT;

  // This lane's X pieces: instruction j of the wave covers tile row
  // rr(j) = rr0 + j * RPI, 16 bytes at piece `piece`; rows past B repeat row
  // B-1 (not stored).  Addresses are formed at each use (holding them would
  // cost 24 VGPRs).
  const int piece = lane % L::PIECES;
  const int rr0 = wave * L::XI_W * L::RPI + lane / L::PIECES;
  const uint16_t *xlane = X + piece * 8;

  u32x4 xr[D][L::XI_W], pr[D][L::PI_HI];
  // Loads of chunk c (clamped to the last chunk, so every set is always
  // filled; pieces past the slice end read the zero block).
  auto load = [&](int set, int c) {
    const int k0 = k_begin + min(c, nchunks - 1) * KC;
    const int k = k0 + piece * 8;
#pragma unroll
    for (int j = 0; j < L::XI_W; ++j) {
      const int row = min(row0 + rr0 + j * L::RPI, B - 1);
      const uint16_t *src = k < k_end ? xlane + (size_t)row * K + k0 : zero;
      xr[set][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
    }
    const int kstep0 = k0 / 32;
#pragma unroll
    for (int j = 0; j < L::PI_HI; ++j) {
      const int inst = j * W + wave;
      if (inst < L::PI)  // wave-uniform
        pr[set][j] = load16(phip + ((size_t)(kstep0 * L::PB + inst) * 64 + lane) * 8);
    }
  };
  auto stash = [&](int set) {
#pragma unroll
    for (int j = 0; j < L::XI_W; ++j) {
      const int rr = rr0 + j * L::RPI;
      *reinterpret_cast<u32x4 *>(lds + rr * L::ROW_BYTES + ((piece ^ (rr & 15)) * 16)) = xr[set][j];
    }
#pragma unroll
    for (int j = 0; j < L::PI_HI; ++j) {
      const int inst = j * W + wave;
      if (inst < L::PI)
        *reinterpret_cast<u32x4 *>(lds + L::X_BYTES + inst * 1024 + lane * 16) = pr[set][j];
    }
  };

  f32x4 acc[L::NB], gram = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < L::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Ops {
    bf16x8 b[L::PB];
    bf16x8 a;
  };
  const int rr_a = wave * 16 + m;
  auto read_ops = [&](Ops &o, int t) {
#pragma unroll
    for (int j = 0; j < L::PB; ++j)
      o.b[j] = *reinterpret_cast<const bf16x8 *>(lds + L::X_BYTES + (t * L::PB + j) * 1024 + lane * 16);
    const int slot = (4 * t + g) ^ m;  // rr_a & 15 == m
    o.a = *reinterpret_cast<const bf16x8 *>(lds + rr_a * L::ROW_BYTES + slot * 16);
  };
  auto mfma_ops = [&](const Ops &o) {
#pragma unroll
    for (int nb = 0; nb < L::NB; ++nb)
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a, o.b[nb], acc[nb], 0, 0, 0);
    gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a, o.a, gram, 0, 0, 0);
  };

#pragma unroll
  for (int d = 0; d < D; ++d) load(d, d);

  for (int c = 0; c < nchunks; c += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int cc = c + d;
      if (cc < nchunks) {  // workgroup-uniform
        // Every wave has finished reading the slots (its MFMAs consumed the
        // reads), so they may be overwritten.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        stash(d);
        wait_lgkmcnt0();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // chunk cc is in LDS
        asm volatile("" ::: "memory");
        load(d, cc + D);
        Ops ops[2];
        read_ops(ops[0], 0);
#pragma unroll
        for (int t = 0; t < L::T; ++t) {
          if (t + 1 < L::T) read_ops(ops[(t + 1) & 1], t + 1);
          __builtin_amdgcn_sched_barrier(0);
          mfma_ops(ops[t & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // D layout of the 16x16 MFMA: lane (m, g) holds rows 4g..4g+3 of column m.
  float *wsl = ws + (size_t)s * B * L::NP;
  const int rbase = row0 + wave * 16;
#pragma unroll
  for (int nb = 0; nb < L::NB; ++nb) {
    const int col = nb * 16 + m;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = rbase + 4 * g + v;
      if (row < B && col < L::N) wsl[(size_t)row * L::NP + col] = acc[nb][v];
    }
  }
  if (g == (m >> 2)) {  // Gram diagonal (m, m): lane (m, m/4), element m%4
    const int row = rbase + m;
    if (row < B) wsl[(size_t)row * L::NP + L::N] = gram[m & 3];
  }
}

}  // namespace

template <int NS, int MB, int KC, int STAGES, int XB, int P2, int W>
hipError_t launch_gemm_lds_typed(const GemmPlan &p, int64_t B, int64_t C, const void *X,
                                 const void *phi, void *ws_base, hipStream_t st) {
  using L = LdsTile<NS, MB, KC, STAGES, XB, P2, W>;
  if (p.row_tiles * L::RT < B) return hipErrorInvalidValue;  // the plan's tiles must cover B
  const int K = (int)(NS * C);
  char *base = static_cast<char *>(ws_base);
  uint16_t *phip = reinterpret_cast<uint16_t *>(base + p.phip_offset);
  uint16_t *zero = reinterpret_cast<uint16_t *>(base + p.zero_offset);
  const int64_t ksteps = (int64_t)(p.phip_bytes / ((size_t)L::PB * 1024));
  hipError_t e;
  if constexpr (P2 == 2) {
    e = launch_pack_phi32(NS, K, ksteps, phi, phip, zero, st);
  } else {
    e = launch_pack_phi(NS, K, ksteps, phi, phip, zero, st);
  }
  if (e != hipSuccess) return e;
  const dim3 grid((uint32_t)p.row_tiles, (uint32_t)p.split);
  gemm_rms_lds_kernel<NS, MB, KC, STAGES, XB, P2, W><<<grid, W * 64, 0, st>>>(
      static_cast<const uint8_t *>(X), phip, zero, reinterpret_cast<float *>(base), (int)B, K,
      (int)p.kslice);
  return hipGetLastError();
}

template <int NS, int W, int KC, int D>
hipError_t launch_gemm_xreg_typed(const GemmPlan &p, int64_t B, int64_t C, const void *X, const void *phi,
                                  void *ws_base, hipStream_t st) {
  using L = XrTile<NS, W, KC>;
  if (p.row_tiles * L::RT < B || p.kc != KC || p.kslice % KC != 0) return hipErrorInvalidValue;
  const int K = (int)(NS * C);
  char *base = static_cast<char *>(ws_base);
  uint16_t *phip = reinterpret_cast<uint16_t *>(base + p.phip_offset);
  uint16_t *zero = reinterpret_cast<uint16_t *>(base + p.zero_offset);
  const int64_t ksteps = (int64_t)(p.phip_bytes / ((size_t)L::PB * 1024));
  hipError_t e = launch_pack_phi(NS, K, ksteps, phi, phip, zero, st);
  if (e != hipSuccess) return e;
  const dim3 grid((uint32_t)p.row_tiles, (uint32_t)p.split);
  gemm_rms_xreg_kernel<NS, W, KC, D><<<grid, W * 64, 0, st>>>(
      static_cast<const uint16_t *>(X), phip, zero, reinterpret_cast<float *>(base), (int)B, K, (int)p.kslice);
  return hipGetLastError();
}

// Instantiations used by the library (see plan_gemm in mhc_gemm_rms.hip).
template hipError_t launch_gemm_lds_typed<1, 1, 256, 3, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
// bf16 X in 128-k chunks, deeper rings (tuning: MHC_GEMM_KC = 128, MHC_GEMM_STAGES)
template hipError_t launch_gemm_lds_typed<1, 1, 128, 5, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<2, 1, 128, 5, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<4, 1, 128, 5, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<1, 1, 128, 6, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<2, 1, 128, 6, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<4, 1, 128, 6, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<2, 1, 256, 3, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<4, 1, 256, 3, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<8, 2, 128, 3, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<8, 2, 256, 2, 1, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<8, 1, 256, 2, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<8, 1, 128, 4, 2, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<1, 1, 256, 4, 1, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<2, 1, 256, 4, 1, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<4, 1, 256, 4, 1, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<8, 1, 256, 2, 1, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<1, 2, 256, 3, 1, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<2, 2, 256, 3, 1, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<4, 2, 256, 3, 1, 1>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
// eight waves per workgroup (128-row tiles)
template hipError_t launch_gemm_lds_typed<1, 1, 128, 4, 2, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<2, 1, 128, 4, 2, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<4, 1, 128, 4, 2, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<1, 1, 256, 2, 2, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<2, 1, 256, 2, 2, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<4, 1, 256, 2, 2, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<8, 1, 128, 3, 2, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<1, 1, 256, 3, 1, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<2, 1, 256, 3, 1, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<4, 1, 256, 3, 1, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<8, 1, 256, 2, 1, 1, 8>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
// X and phi through registers (bf16 X at n = 8)
template hipError_t launch_gemm_xreg_typed<8, 8, 256, 2>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_xreg_typed<4, 8, 256, 2>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
// fp32 phi (hi + lo parts)
template hipError_t launch_gemm_lds_typed<1, 1, 128, 4, 2, 2>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<2, 1, 128, 4, 2, 2>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<4, 1, 128, 4, 2, 2>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);
template hipError_t launch_gemm_lds_typed<8, 1, 128, 2, 2, 2>(const GemmPlan &, int64_t, int64_t, const void *, const void *, void *, hipStream_t);

}  // namespace mhc
