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
//            copy of phi_{t+1} (see mhc_pack.hip; in the fixed-slice layout
//            gathered from phi_{t+1} itself once per run and held in
//            registers, with no packing launch) and
//            accumulates v_mfma_f32_16x16x32_bf16 plus the Gram block for the
//            sum of squares;
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
//
// Pre-mix mode (kFusedApplyPreBf16 / kFusedApplyPreFp8, n <= 4,
// mhc_post_res_coeffs_pre / mhc_post_res_coeffs_pre_fp8).  The
// next layer also needs F_pre = sum_i H_pre[i] X_{t+1}[i] (section 2.5,
// first step), and H_pre needs the whole row's product (sections 2.1-2.4),
// which S workgroups compute slice by slice.  This mode forms F_pre in the
// same pass, so X_{t+1} is written once and never read back at all:
//   * one step per unit (a unit's flush is its total) and a grid of whole
//     row tiles (G % S == 0): the S slices of a row tile are always taken
//     in the same round by S co-resident workgroups;
//   * two LDS tiles: step t's X_{t+1} rows stay on chip until step t+2
//     rewrites their tile;
//   * at the start of step t+1 each workgroup publishes, per row of step t,
//     the n pre logits and the sum of squares of its slice as 4-byte
//     records in the workspace (buffer stores with the SC1 bit, which the
//     gfx950 memory model uses for agent-scope coherence across XCDs; a
//     record is zero until written, and a written value is never the zero
//     word: +0.0 is stored as -0.0);
//   * at step t+2 each wave reads its row's records for all S slices (one
//     8-byte load per lane, issued at the start of the step, checked after
//     the apply; a rare miss is polled with a bounded wait), sums each
//     column over 16 slice slots as a balanced tree (the order the combine
//     kernel uses in this mode, so H_pre comes out bitwise as in H_next),
//     forms the n gates and emits its row of F_pre from the tile exactly as
//     pre_kernel would from X_{t+1} in HBM (E4M3: the tile holds the E4M3
//     values widened exactly, so the same chain gives pre_fp8_kernel's bits;
//     the product-only E4M3 mode keeps its X values in registers instead).
// No workgroup waits for one that has not started: a wait at step t+2 needs
// only records published at the start of step t+1 by workgroups of the same
// round, and every workgroup publishes before it waits (induction over t;
// all G workgroups are resident at once: the host sizes G from the
// occupancy the runtime reports and the compute units of the stream).  A
// wait that still cannot end (e.g. kernels on other streams hold CUs) gives
// up after about a second, writes NaN to its F_pre vector and sets the
// give-up word of the workspace, which the caller can read back
// (mhc_post_res_coeffs_pre_check).
//
// The first layer has no apply: its X_t is the stream built from the
// embeddings.  The product-only pre-mix modes (kFusedCoeffsPreBf16 /
// kFusedCoeffsPreFp8, mhc_coeffs_pre / mhc_coeffs_pre_fp8) run the same pass
// on X_t itself: X_t goes into the tiles as read, nothing is written back,
// and F_pre = sum_i H_pre[i] X_t[i] comes out of the same hand-off, so the
// first layer also reads its stream once.
#include "mhc_device.h"
#include "mhc_finish.h"
#include "mhc_launch.h"

#include <atomic>
#include <cstdlib>
#include <type_traits>

namespace mhc {

namespace {

constexpr int kStepCh = 512;          // channels per step: 64 lanes x 8
constexpr int kLdsMax = 160 * 1024;   // LDS of one CU

// Pre-mix mode: a hand-off record is one fp32 value in 4 bytes.  The records
// are zero-filled before every launch and a stored value is never the zero
// word (+0.0 is stored as -0.0), so a record holds either zero (not yet
// written) or its value, written by one single-copy-atomic store.
constexpr uint32_t kRecNegZero = 0x80000000u;
// Bound on the polls of one wait for records (each poll sleeps ~0.2 us and
// reads memory): a wait that cannot end, e.g. when the grid is not fully
// resident, gives up after well under a second and poisons its outputs.
constexpr int kSpinLimit = 1 << 17;
// Word 3 of a gfx9 buffer resource for raw (untyped) access, and the cache
// policy bit SC1 of a buffer access (agent-scope coherence, as the compiler
// gives agent-scope atomic loads and stores).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kSc1 = 16;

template <int NS, bool PRE = false>
struct FusedTile {
  static constexpr int N = NS * NS + 2 * NS;
  static constexpr int NP = N + 1;
  static constexpr int NB = (N + 15) / 16;
  // Rows per tile = waves per workgroup (one workgroup per CU).  A tile of
  // R < 16 rows would repeat its rows in the upper MFMA rows (results there
  // unused); 8-row tiles with two workgroups per CU measured slower for the
  // pre-mix mode (twice the phi operand traffic per row).
  static constexpr int R = 16;
  static constexpr int THREADS = 64 * R;
  static constexpr int ROW_BYTES = NS * kStepCh * 2;   // one tile row in LDS
  static constexpr int TILE_BYTES = R * ROW_BYTES;     // 64 KiB at n=4, 128 KiB at n=8 (R = 16)
  static constexpr int NT = PRE ? 2 : 1;               // tiles (pre-mix: this step's and the one before)
  static constexpr int KSTEPS = 16 * NS;               // 32-channel MFMA steps per step
  static constexpr int KPW = KSTEPS / R;               // ... per wave
  static constexpr int KB = NS >= 8 ? 2 : (KPW < 4 ? KPW : 4);  // k-steps whose B operands are held at once
  static constexpr int NH = NS + NS * NS;              // H_post and H_res of one row
  static constexpr int HV = (NH + 63) / 64;            // dwords per lane that hold them
  // Reduction rows: the NB*16 product columns, then the Gram sum; the
  // pre-mix mode puts the Gram sum in the last padding column (N < NB*16)
  // so that the two tiles and the buffer fit 160 KiB at n = 4.
  static constexpr int GRAM_COL = PRE ? NB * 16 - 1 : NB * 16;
  static constexpr int RS = PRE ? NB * 16 : NB * 16 + 1;
  static constexpr int RED_BYTES = R * 16 * RS * 4;    // [R waves][16 MFMA rows][RS] fp32
  // The reduction buffer sits beside the tile when both fit (then the flush
  // of step s-1 overlaps step s); otherwise it reuses the tile buffer.
  static constexpr bool SEPARATE = NT * TILE_BYTES + RED_BYTES <= kLdsMax;
  static constexpr int LDS_BYTES = SEPARATE ? NT * TILE_BYTES + RED_BYTES
                                            : (TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES);
  static constexpr int OPT = (R * NP + THREADS - 1) / THREADS;  // flushed sums per thread
  // Pre-mix hand-off: per (row, slice) the n pre logits and the sum of
  // squares, padded to an even count PW of 4-byte records; one 8-byte load
  // per lane reads a row's records for up to 16 slices (16 * PW <= 128).
  static constexpr int PW = (NS + 2) & ~1;
  static constexpr int RB = NS >= 4 ? 2 : 1;  // 16-lane column groups needed: n + 1 columns
  static_assert(LDS_BYTES <= kLdsMax, "LDS budget");
  static_assert(!PRE || (SEPARATE && N < NB * 16), "pre-mix mode needs n <= 4");
};

struct Step {
  int row0, c0, c_end, slot;
};

// What the kernel reads, writes and multiplies (FusedMode, mhc_launch.h).
template <int MODE>
struct FusedIO {
  static constexpr bool FP8 = MODE == kFusedApplyFp8 || MODE == kFusedCoeffsFp8 || MODE == kFusedApplyPreFp8 ||
                             MODE == kFusedCoeffsPreFp8;
  static constexpr bool PRE = is_pre_mode(MODE);
  static constexpr bool APPLY_BF16 = MODE == kFusedApplyBf16 || MODE == kFusedApplyPreBf16;
  static constexpr bool APPLY_FP8 = MODE == kFusedApplyFp8 || MODE == kFusedApplyPreFp8;
  static constexpr bool APPLY = APPLY_BF16 || APPLY_FP8;
  static constexpr int EB = FP8 ? 1 : 2;  // bytes per element
  using vec = typename std::conditional<FP8, u32x2, u32x4>::type;  // 8 elements per lane
};

// FIX: the fixed-slice layout (one step per unit, a grid of whole row tiles,
// n <= 4; always so in the pre-mix mode), in which a workgroup keeps one
// slice for its whole run.
template <int NS, int MODE, bool FIX>
__global__ __launch_bounds__(1024) void post_res_next_kernel(
    const uint8_t *__restrict__ X, const uint8_t *__restrict__ F, const float *__restrict__ H,
    uint8_t *__restrict__ Y, const uint16_t *__restrict__ phip, float *__restrict__ ws,
    float *__restrict__ dummy, int B, int C, int spu, int S, int U, const PreArgs pa) {
  using IO = FusedIO<MODE>;
  using T = FusedTile<NS, IO::PRE>;
  using vec = typename IO::vec;
  // F_pre from register-held E4M3 values (the product-only E4M3 pre-mix
  // mode) rather than from the tile.
  constexpr bool KV = IO::PRE && IO::FP8 && !IO::APPLY;
  static_assert(!IO::PRE || FIX, "the pre-mix mode runs the fixed-slice layout");
  static_assert(!FIX || T::KB == T::KPW, "the fixed-slice layout holds every k-step's operands");
  __shared__ __attribute__((aligned(1024))) char lds[T::LDS_BYTES];
  float *red = reinterpret_cast<float *>(lds + (T::SEPARATE ? T::NT * T::TILE_BYTES : 0));

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

  // The fixed-slice layout has one step per unit and a grid of whole row
  // tiles (G % S == 0), so a workgroup keeps one slice and its row tile
  // advances by G/S tiles per step: no division per step.
  [[maybe_unused]] const int pre_slot = uniform(pg % S), pre_tile0 = uniform(pg / S), pre_gs = uniform(G / S);
  auto step_at = [&](int t) {
    if constexpr (FIX) {
      const int cb = pre_slot * kStepCh;
      return Step{uniform((t * pre_gs + pre_tile0) * T::R), cb, uniform(min(C, cb + kStepCh)), pre_slot};
    } else {
      const int j = t / spu, p = t - j * spu;
      const int u = j * G + pg;
      const int tile = u / S, s = u - tile * S;
      const int cb = s * cw;
      return Step{uniform(tile * T::R), uniform(cb + p * kStepCh), uniform(min(C, cb + cw)), uniform(s)};
    }
  };

  // The tile of step t (the pre-mix mode alternates two).
  auto tile_of = [&](int t) -> char * { return lds + (IO::PRE ? (t & 1) * T::TILE_BYTES : 0); };
  const int wslot = (lane ^ (wave & 15)) * 16;  // swizzled 16-byte slot of this lane
  // Buffer resources of the pre-mix mode (gfx9 raw buffers: stride 0, the
  // size in bytes as the record count; accesses past it are dropped).
  [[maybe_unused]] __amdgpu_buffer_rsrc_t ws_rsrc, rec_rsrc, phi_rsrc;
  [[maybe_unused]] const uint32_t lane_off16 = (uint32_t)lane * 16u;
  if constexpr (FIX)
    phi_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(pa.phi), (short)0, (int)pa.phi_bytes, kRsrcWord3);
  if constexpr (IO::PRE) {
    ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(ws, (short)0, (int)pa.partial_bytes, kRsrcWord3);
    rec_rsrc = __builtin_amdgcn_make_buffer_rsrc(pa.rec, (short)0, (int)pa.rec_bytes, kRsrcWord3);
  }

  // In the fixed-slice layout (KB = KPW at n <= 4) the phi operands of each
  // wave's k-steps are the same on every step: gathered once here straight
  // from phi [K, N] and held in registers.  Lane (m, g) of k-step ks and
  // column block nb takes phi[32 ks + 8 g + j][16 nb + m], j = 0..7 (the
  // B operand layout of v_mfma_f32_16x16x32_bf16); columns past N read past
  // the buffer, i.e. zero.
  [[maybe_unused]] bf16x8 bfix[FIX ? T::KB : 1][T::NB];
  if constexpr (FIX) {
    const int cb = pre_slot * kStepCh;
#pragma unroll
    for (int q = 0; q < T::KB; ++q) {
      const int ks = wave * T::KPW + q;
      const int i = ks >> 4, ts = ks & 15;
      const int kstep = (i * C + min(cb + 32 * ts, C - 32)) >> 5;  // clamped in range; such steps add zero
#pragma unroll
      for (int nb = 0; nb < T::NB; ++nb) {
        const int col = nb * 16 + m;
        const uint32_t base = col < T::N ? (uint32_t)((kstep * 32 + 8 * g) * T::N + col) * 2u : 0x80000000u;
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(phi_rsrc, base + (uint32_t)(2 * h * T::N * 2), 0, 0);
          const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(phi_rsrc, base + (uint32_t)((2 * h + 1) * T::N * 2), 0, 0);
          w[h] = lo | (hi << 16);
        }
        bfix[q][nb] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
      }
    }
  }

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
  // unit's partials.  Threads without a target write the dummy area; so
  // does everything when `real` is false (the flush before the first step).
  // The pre-mix mode also publishes the n pre logits and the sum of squares
  // as tagged records: one 8-byte store each, value and tag together, which
  // another workgroup can read without any ordering between stores.
  auto flush = [&](const Step &sp, bool real) {
#pragma unroll
    for (int q = 0; q < T::OPT; ++q) {
      const int e = tid + q * T::THREADS;
      const int ec = min(e, T::R * T::NP - 1);
      const int r = ec / T::NP, col = ec - r * T::NP;
      const int rcol = col < T::N ? col : T::GRAM_COL;
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < T::R; ++w) a += red[(w * 16 + r) * T::RS + rcol];
      const int row = sp.row0 + r;
      const bool tgt = real && e < T::R * T::NP && row < B;
      if constexpr (!IO::PRE) {
        float *dst = tgt ? ws + ((size_t)sp.slot * B + row) * T::NP + col : dummy + e;
        *dst = a;
      } else {
        // Buffer stores: a thread without a target stores past the buffer
        // (dropped).  The record is one 8-byte store with the SC1 bit (the
        // agent-scope coherence of the gfx950 memory model), value and tag
        // together.
        constexpr uint32_t kNone = 0x80000000u;
        const uint32_t poff = tgt ? (uint32_t)((sp.slot * B + row) * T::NP + col) * 4u : kNone;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), ws_rsrc, poff, 0, 0);
        const bool rec = tgt && (col < NS || col == T::N);
        const int rc = col < NS ? col : NS;
        const uint32_t roff = rec ? (uint32_t)((row * S + sp.slot) * T::PW + rc) * 4u : kNone;
        const uint32_t bits = __float_as_uint(a);
        __builtin_amdgcn_raw_buffer_store_b32(bits == 0u ? kRecNegZero : bits, rec_rsrc, roff, 0, kSc1);
      }
    }
  };

  auto write_red = [&]() {
    float *rw = red + wave * 16 * T::RS;
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) rw[(4 * g + v) * T::RS + nb * 16 + m] = acc[nb][v];
    // (In the pre-mix mode this lands on a padding column written just above
    // by the same wave; the later write wins.)  The empty asm makes the lane
    // index opaque, so the address is formed here rather than hoisted out of
    // the step loop (where, in the pre-mix mode, it was spilled to scratch,
    // and reloading it waited for every load in flight).
    int mm = m;
    if constexpr (IO::PRE) asm volatile("" : "+v"(mm));
    if (g == (mm >> 2)) rw[mm * T::RS + T::GRAM_COL] = gram[mm & 3];
  };

  // ---- pre-mix mode: F_pre of the next layer, two steps behind the apply.
  // Step q's X_{t+1} rows stay in their LDS tile until step q+2 (or the end)
  // rewrites it.  By then every slice of q's row tile has (normally) been
  // flushed by its workgroup, so the row's n pre logits and sum of squares
  // can be summed in slice order 0..S-1 -- the order of the combine kernel,
  // hence the same H_pre bits -- and F_pre[row, chunk] = sum_i H_pre[i]
  // X_{t+1}[i, chunk] is formed from the tile exactly as pre_kernel forms it.
  // b_pre of the gate lane 16i forms (lanes past the n columns: any valid one)
  [[maybe_unused]] float bpre_lane = 0.f;
  if constexpr (IO::PRE) bpre_lane = pa.b_pre[min(lane >> 4, NS - 1)];
  // Records of step q's row for this wave ([B][S][PW] words: a row's records
  // are contiguous): lane l reads words 2l, 2l+1, i.e. slice 2l / PW; lanes
  // past the row read past the buffer (zeros, never checked).  Agent scope
  // (SC1): served past this XCD's L2, where another XCD's stores land.
  using rec_t = u32x2;
  auto rec_load = [&](rec_t &rv, int q) {
    const Step sp = step_at(q);
    const int rr = uniform(min(sp.row0 + wave, B - 1));
    const uint32_t off = 2 * lane < S * T::PW ? (uint32_t)(rr * S * T::PW + 2 * lane) * 4u : 0x80000000u;
    rv = __builtin_amdgcn_raw_buffer_load_b64(rec_rsrc, off, 0, kSc1);
  };
  auto rec_ready = [&](const rec_t &rv) -> bool {
    const int w = 2 * lane;                       // first word of this lane
    const bool lo_used = w < S * T::PW && (w % T::PW) <= NS;
    const bool hi_used = w + 1 < S * T::PW && ((w + 1) % T::PW) <= NS;
    const bool ok = (!lo_used || rv[0] != 0u) && (!hi_used || rv[1] != 0u);
    return __builtin_amdgcn_ballot_w64(!ok) == 0;
  };
  // Poll until every record is there; true if the wait gave up.
  auto rec_wait = [&](rec_t &rv, int q) -> bool {
    if (rec_ready(rv)) return false;
    bool ready = false;
    int tries = 0;
    do {
      __builtin_amdgcn_s_sleep(8);
      rec_load(rv, q);
      ready = rec_ready(rv);
    } while (!ready && ++tries < kSpinLimit);
    return !ready;
  };
  // H_pre of the row from its records.  Lane 16c + s gathers column c of
  // slice s (word s*PW + c, in lane (s*PW + c)/2, half c&1; zero past S) and
  // each 16-lane group sums its column over the 16 slice slots as a
  // balanced binary tree (tree16_sum), the order the combine kernel uses in
  // this mode: equal sums, equal H_pre bits.  Lane 16i then forms gate i.
  auto pre_coeffs = [&](const rec_t &rv, float (&hp)[NS]) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // keep the gather addresses out of the loop's live registers
    const int sl = ln & 15;
    float t[T::RB];
#pragma unroll
    for (int b = 0; b < T::RB; ++b) {
      const int c = b == 0 ? min(ln >> 4, NS) : NS;  // column of this lane's group
      const int src = (sl * T::PW + c) >> 1;
      const int lo = __builtin_amdgcn_ds_bpermute(src * 4, (int)rv[0]);
      const int hi = __builtin_amdgcn_ds_bpermute(src * 4, (int)rv[1]);
      const float v = __int_as_float((c & 1) ? hi : lo);
      t[b] = tree16_sum(sl < S ? v : 0.f);
    }
    const float sq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t[T::RB - 1]), NS < 4 ? 16 * NS : 0));
    const float inv_r = recip_exact(row_rms(sq, pa.inv_k));
    const float gate = pre_gate(t[0], inv_r, pa.alpha_pre, bpre_lane);
#pragma unroll
    for (int i = 0; i < NS; ++i) hp[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gate), 16 * i));
  };
  // F_pre of this wave's row of step q, from the row's tile (bf16; in the
  // E4M3 apply mode the E4M3 values widened exactly, so the fp32 chain below
  // sees the values pre_fp8_kernel widens from E4M3), or in the product-only
  // E4M3 mode (KV) from kv, this lane's own X values of step q (kept in
  // registers for two steps).  `real` false (before the first step) or a row
  // past B gives the store an empty buffer (dropped); a given-up wait
  // poisons the vector with NaN.  Lanes past the slice take the last in-range
  // vector's tile slot or computed the owning lane's values from clamped
  // addresses, so they store the owning lane's bytes to the owning lane's
  // address.
  auto emit = [&](int q, const float (&hp)[NS], bool poison, bool real, const vec (&kv)[NS]) {
    const Step sp = step_at(q);
    if (poison) {
      // Report the give-up (a vector buffer store, agent scope; every lane
      // stores the same word).
      const __amdgpu_buffer_rsrc_t frs = __builtin_amdgcn_make_buffer_rsrc(pa.giveup, (short)0, 4, kRsrcWord3);
      __builtin_amdgcn_raw_buffer_store_b32(1u, frs, 0u, 0, kSc1);
    }
    const int row = sp.row0 + wave;
    const int cst = min(sp.c0 + 8 * lane, sp.c_end - 8);
    // fp32 FMA chain over the streams in stream order from zero, one rounding
    // at the end: pre_kernel's arithmetic (pre_fp8_kernel's for E4M3).
    float a[8];
    if constexpr (KV) {
      // The E4M3 values themselves, widened to fp32 (exact), two per instruction.
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const f32x2 lo = fp8_lo2(kv[j][d]), hi = fp8_hi2(kv[j][d]);
          s4[0] = fmaf(hp[j], lo[0], s4[0]);
          s4[1] = fmaf(hp[j], lo[1], s4[1]);
          s4[2] = fmaf(hp[j], hi[0], s4[2]);
          s4[3] = fmaf(hp[j], hi[1], s4[3]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) a[4 * d + k] = s4[k];
      }
    } else {
      // The lane's 16-byte slot of its row of the tile.
      const int slot = (((cst - sp.c0) >> 3) ^ (wave & 15)) * 16;
      const char *src = tile_of(q) + wave * T::ROW_BYTES;
      u32x4 xv[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) xv[i] = *reinterpret_cast<const u32x4 *>(src + i * (kStepCh * 2) + slot);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          a0 = fmaf(hp[j], bf16_lo(xv[j][w]), a0);
          a1 = fmaf(hp[j], bf16_hi(xv[j][w]), a1);
        }
        a[2 * w] = a0;
        a[2 * w + 1] = a1;
      }
    }
    // The row's own buffer; a row without a target (past B, or before the
    // first step) gets an empty one, so the store is dropped.  Cache policy
    // by mode, as measured at n=4, C=7168, B=16384: after the apply the
    // default one (412-417 against 439-442 us per call with the streaming
    // bit); in the product-only modes (the first layer) the streaming one
    // (217.5-218.2 against 223.8-225.1 us in bf16; E4M3 unchanged).
    constexpr int kFpreAux = IO::APPLY ? 0 : 2;
    const bool tgt = real && row < B;  // wave-uniform
    const __amdgpu_buffer_rsrc_t frow = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint8_t *>(pa.F_pre) + (size_t)min(row, B - 1) * C * IO::EB, (short)0,
        tgt ? C * IO::EB : 0, kRsrcWord3);
    if constexpr (IO::FP8) {
      u32x2 o{pack_fp8x4(a[0], a[1], a[2], a[3]), pack_fp8x4(a[4], a[5], a[6], a[7])};
      if (poison) o = u32x2{0x7f7f7f7fu, 0x7f7f7f7fu};  // E4M3 NaN
      __builtin_amdgcn_raw_buffer_store_b64(o, frow, (uint32_t)cst, 0, kFpreAux);
    } else {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = pack_bf16x2(a[2 * w], a[2 * w + 1]);
      if (poison) o = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
      __builtin_amdgcn_raw_buffer_store_b128(o, frow, (uint32_t)cst * 2u, 0, kFpreAux);
    }
  };

  // One step on the loads in (xv, fv, hv); refills them with step t_pref.
  auto step = [&](int t, vec (&xv)[NS], vec &fv, uint32_t (&hv)[T::HV], int t_pref, vec (&kv)[NS]) {
    const Step sp = step_at(t);
    [[maybe_unused]] u32x2 rv;
    if constexpr (IO::PRE) {
      // The pre-mix mode publishes step t-1's sums first thing, a whole step
      // before any workgroup reads them (at step t+1), and issues the reads
      // of step t-2's records ahead of its own stores, so checking them after
      // the apply waits for no store of this step.
      __syncthreads();  // red holds step t-1's sums
      rec_load(rv, t >= 2 ? t - 2 : 0);
      flush(step_at(t > 0 ? t - 1 : 0), t > 0);
    }
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
    if constexpr (IO::APPLY_BF16) {
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
    } else if constexpr (IO::APPLY_FP8) {
      // E4M3: each 8-byte vector is two words of four channels; the same
      // arithmetic per element as post_res_fp8_kernel (at n = 4 the mix on
      // the matrix core, mix4_pair; otherwise an FMA chain), then the E4M3
      // result is widened (exactly) for the tile.
      if constexpr (NS == 4) {
        // Row (lane & 3) of H_res and H_post[lane & 3] from the lanes of hv.
        const int i4 = lane & 3;
        auto bperm = [&](int src) { return __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, (int)hv[0])); };
        const Mix4A ma = mix4_a(bperm(NS + i4 * NS), bperm(NS + i4 * NS + 1), bperm(NS + i4 * NS + 2),
                                bperm(NS + i4 * NS + 3), bperm(i4));
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          f32x4 v0, v1;
          mix4_pair(ma, xv[0][d], xv[1][d], xv[2][d], xv[3][d], fv[d], 0, v0, v1);
#pragma unroll
          for (int i = 0; i < NS; ++i) out[i][d] = pack_fp8x2_lo(v0[i], v1[i]);
          mix4_pair(ma, xv[0][d], xv[1][d], xv[2][d], xv[3][d], fv[d], 2, v0, v1);
#pragma unroll
          for (int i = 0; i < NS; ++i) out[i][d] = pack_fp8x2_hi(out[i][d], v0[i], v1[i]);
        }
      } else if constexpr (NS <= 4) {
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
      if constexpr (IO::APPLY_BF16) return out[i];
      else if constexpr (IO::APPLY_FP8) return fp8x8_to_bf16(out[i]);
      else if constexpr (IO::FP8) return fp8x8_to_bf16(xv[i]);  // the product-only E4M3 modes
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
        for (int nb = 0; nb < T::NB; ++nb) {
          if constexpr (FIX)
            b[q][nb] = bfix[q][nb];
          else
            b[q][nb] = __builtin_bit_cast(bf16x8, load16(phip + ((size_t)(kstep * T::NB + nb) * 64 + lane) * 8));
        }
      }
    };
    char *my_lds_row = tile_of(t) + wave * T::ROW_BYTES;
    if constexpr (IO::PRE) {
      if constexpr (IO::APPLY) {
        uint8_t *yr = Y + (size_t)rr * NS * C * IO::EB;
#pragma unroll
        for (int i = 0; i < NS; ++i)
          __builtin_nontemporal_store(out[i], reinterpret_cast<vec *>(yr + ((size_t)i * C + cst) * IO::EB));
      }
      // Keep the record check below the stores: the check's wait then covers
      // only loads issued at least a step ago (and the step's own stores).
      load_b(0);
      asm volatile("" ::: "memory");
      // F_pre of step t-2 from this wave's row of tile t&1, then this step's
      // row into the same place (the wave's own row: program order suffices;
      // every wave finished reading tile t&1 for step t-2's product before
      // the barriers of step t-1).
      const bool have = t >= 2;
      bool poison = false;
      if (have) poison = rec_wait(rv, t - 2);
      float hp[NS];
      pre_coeffs(rv, hp);
      emit(have ? t - 2 : 0, hp, poison, have, kv);
      if constexpr (KV) {
#pragma unroll
        for (int i = 0; i < NS; ++i) kv[i] = xv[i];  // this step's X, emitted two steps on
      }
#pragma unroll
      for (int i = 0; i < NS; ++i)
        *reinterpret_cast<u32x4 *>(my_lds_row + i * (kStepCh * 2) + wslot) =
            (in_range && live) ? tile_vec(i) : u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (IO::APPLY && !IO::PRE) {
      uint8_t *yr = Y + (size_t)rr * NS * C * IO::EB;
#pragma unroll
      for (int i = 0; i < NS; ++i)
        __builtin_nontemporal_store(out[i], reinterpret_cast<vec *>(yr + ((size_t)i * C + cst) * IO::EB));
    }
    // The first B group is issued before the refill (waiting for it then
    // never waits for the refill), except for n = 8, where holding it across
    // the refill would not fit the register budget.
    if constexpr (NS < 8 && !IO::PRE) load_b(0);

    if constexpr (!IO::PRE) {
      __syncthreads();  // the previous step's product is done with the tile (and has written red)
      if constexpr (T::SEPARATE) flush(step_at(t > 0 ? t - 1 : 0), t > 0);
#pragma unroll
      for (int i = 0; i < NS; ++i)
        *reinterpret_cast<u32x4 *>(my_lds_row + i * (kStepCh * 2) + wslot) =
            (in_range && live) ? tile_vec(i) : u32x4{0u, 0u, 0u, 0u};
    }
    load_set(xv, fv, hv, step_at(t_pref));
    if constexpr (NS >= 8) load_b(0);
    __syncthreads();  // the tile is complete (and the flush has read red)

    // A unit's sums start from zero at its first step (every step in the
    // fixed-slice layout, which has one step per unit: the sums then live
    // only within the step).
    const bool first = FIX || (t % spu) == 0;
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
        const int rm = m & (T::R - 1);  // tile row of MFMA row m
        const int piece = (4 * ts + g) ^ rm;
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(tile_of(t) + rm * T::ROW_BYTES + i * (kStepCh * 2) + piece * 16);
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
      flush(sp, true);  // the next step's first barrier orders it before the tile is rewritten
    }
  };

  const int tl = nsteps - 1;
  // The product-only E4M3 pre-mix mode's own X values of the last two steps,
  // one set per register set (step t runs on set t & 1: ka for even t, kb
  // for odd).
  [[maybe_unused]] vec ka[NS], kb[NS];
  if constexpr (NS >= 8) {
    // n = 8: one register set (two would not fit 128 VGPRs).
    vec xa[NS], fa;
    uint32_t ha[T::HV];
    load_set(xa, fa, ha, step_at(0));
    for (int t = 0; t < nsteps; ++t) step(t, xa, fa, ha, min(t + 1, tl), ka);
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
      step(t, xa, fa, ha, min(t + 2, tl), ka);
      step(t + 1, xb, fb, hb, min(t + 3, tl), kb);
    }
    if (t < nsteps) step(t, xa, fa, ha, tl, ka);
  }
  if constexpr (T::SEPARATE) {
    __syncthreads();
    flush(step_at(tl), true);
  }
  if constexpr (IO::PRE) {
    // The last two steps' F_pre (their tiles are intact: nothing rewrote them;
    // with KV, step q's own values are in ka or kb by the parity of q).
    auto tail = [&](int q, const vec (&kv)[NS]) {
      u32x2 rv;
      rec_load(rv, q);
      const bool poison = rec_wait(rv, q);
      float hp[NS];
      pre_coeffs(rv, hp);
      emit(q, hp, poison, true, kv);
    };
    if (tl >= 1) {
      if (tl & 1) {
        tail(tl - 1, ka);
        tail(tl, kb);
      } else {
        tail(tl - 1, kb);
        tail(tl, ka);
      }
    } else {
      tail(tl, ka);
    }
  }
}



template <int NS, int MODE, bool FIX>
hipError_t launch_post_res_next_typed(int64_t B, int64_t C, int spu, int split, int G,
                                      const void *X, const void *F, const float *H, void *Y,
                                      const void *phip, float *ws, float *dummy,
                                      const PreArgs &pa, hipStream_t st) {
  using T = FusedTile<NS, FusedIO<MODE>::PRE>;
  const int64_t U = ((B + T::R - 1) / T::R) * (int64_t)split;
  post_res_next_kernel<NS, MODE, FIX><<<dim3((uint32_t)G), T::THREADS, 0, st>>>(
      static_cast<const uint8_t *>(X), static_cast<const uint8_t *>(F), H,
      static_cast<uint8_t *>(Y), static_cast<const uint16_t *>(phip), ws, dummy, (int)B, (int)C,
      spu, split, (int)U, pa);
  return hipGetLastError();
}

template <int NS, int MODE>
hipError_t launch_layout(bool fixed, int64_t B, int64_t C, int spu, int split, int G, const void *X,
                         const void *F, const float *H, void *Y, const void *phip, float *ws,
                         float *dummy, const PreArgs &pa, hipStream_t st) {
  if constexpr (is_pre_mode(MODE)) {
    if (!fixed) return hipErrorInvalidValue;
    return launch_post_res_next_typed<NS, MODE, true>(B, C, spu, split, G, X, F, H, Y, phip, ws, dummy, pa, st);
  } else if constexpr (NS >= 8) {
    if (fixed) return hipErrorInvalidValue;  // n = 8 holds its operands in two groups
    return launch_post_res_next_typed<NS, MODE, false>(B, C, spu, split, G, X, F, H, Y, phip, ws, dummy, pa, st);
  } else {
    return fixed ? launch_post_res_next_typed<NS, MODE, true>(B, C, spu, split, G, X, F, H, Y, phip, ws, dummy, pa, st)
                 : launch_post_res_next_typed<NS, MODE, false>(B, C, spu, split, G, X, F, H, Y, phip, ws, dummy, pa, st);
  }
}

template <int MODE>
hipError_t launch_mode(int n, bool fixed, int64_t B, int64_t C, int spu, int split, int G, const void *X,
                       const void *F, const float *H, void *Y, const void *phip, float *ws,
                       float *dummy, const PreArgs &pa, hipStream_t st) {
  switch (n) {
    case 1: return launch_layout<1, MODE>(fixed, B, C, spu, split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case 2: return launch_layout<2, MODE>(fixed, B, C, spu, split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case 4: return launch_layout<4, MODE>(fixed, B, C, spu, split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case 8:
      if constexpr (is_pre_mode(MODE)) return hipErrorInvalidValue;  // n <= 4 only
      else return launch_layout<8, MODE>(fixed, B, C, spu, split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    default: return hipErrorInvalidValue;
  }
}

constexpr int kRecordSlices = 16;  // slices one record gather covers
constexpr int kPreRows = 16;       // rows per tile of the pre-mix mode (FusedTile::R)

}  // namespace

// Compute units of the current device (cached per device id); declared in
// mhc_launch.h.
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

bool pre_mode_fits(int64_t B, int n, int64_t C) {
  if (n != 1 && n != 2 && n != 4) return false;
  const int64_t steps = (C + kStepCh - 1) / kStepCh;
  const int64_t N = (int64_t)n * n + 2 * n;
  const int64_t lim = int64_t(1) << 31;
  const int64_t phi_bytes = (int64_t)n * C * N * 2;
  return steps <= kRecordSlices && steps <= device_cus() && C * 2 < lim && phi_bytes < lim &&
         steps * B * ((n + 2) & ~1) * 4 < lim && steps * B * (N + 1) * 4 < lim;
}

// The fixed-slice layout: one 512-channel step per unit and a grid of whole
// row tiles, so that each workgroup keeps one slice and holds its phi
// operands in registers for the whole run (n <= 4; n = 8 needs its
// registers for two groups of operands).  It needs one workgroup per slice
// at least and phi addressable by 32-bit buffer offsets.
bool fixed_layout_fits(int n, int64_t C) {
  if (n != 1 && n != 2 && n != 4) return false;
  const int64_t steps = (C + kStepCh - 1) / kStepCh;
  const int64_t N = (int64_t)n * n + 2 * n;
  const int64_t phi_bytes = (int64_t)n * C * N * 2;  // phi itself, addressed by 32-bit buffer offsets
  return steps <= device_cus() && phi_bytes < (int64_t(1) << 31);
}

FusedPlan plan_post_res_next(int64_t B, int n, int64_t C, bool pre, bool prefer_fixed) {
  FusedPlan p;
  const int64_t N = (int64_t)n * n + 2 * n, NB = (N + 15) / 16, K = (int64_t)n * C;
  p.row_tiles = pre ? (B + kPreRows - 1) / kPreRows : (B + 15) / 16;
  p.pre = pre;
  p.fixed = pre;
  if (!pre && fixed_layout_fits(n, C)) {
    p.fixed = prefer_fixed;
    if (tune(kTuneFusedFixed) >= 0) p.fixed = tune(kTuneFusedFixed) != 0;
  }
  // Steps per unit: the largest divisor of the row's step count that still
  // leaves at least 7 slices (fewer when the row is shorter), so that the
  // ~256 resident workgroups cover at most ~37 row tiles at a time while the
  // partial sums stay small (7 x B x (N+1) fp32).  MHC_FUSED_SPU overrides
  // (any value >= 1; one that does not divide the step count leaves empty
  // steps at the end of the last slice, which add nothing).  The pre-mix
  // mode takes one step per unit: a unit's flush is then its total.
  const int64_t steps = (C + kStepCh - 1) / kStepCh;
  const int64_t want = steps < 7 ? steps : 7;
  int64_t spu = 1;
  if (!p.fixed) {
    for (int64_t d = 1; d <= steps; ++d)
      if (steps % d == 0 && steps / d >= want) spu = d;
    const int64_t v = tune(kTuneFusedSpu);
    if (v >= 1 && v <= steps) spu = v;
  }
  p.cw = (int)(spu * kStepCh);
  p.split = (int)((steps + spu - 1) / spu);
  p.partial_bytes = (size_t)p.split * (size_t)B * (size_t)(N + 1) * sizeof(float);
  p.ksteps = (K + 31) / 32;
  p.dummy_offset = (p.partial_bytes + 1023) & ~(size_t)1023;
  p.dummy_bytes = (size_t)((16 * (N + 1) + 1023) / 1024) * 1024 * sizeof(float);
  p.phip_offset = p.dummy_offset + p.dummy_bytes;
  p.phip_bytes = p.fixed ? 0 : (size_t)p.ksteps * (size_t)NB * 1024;  // the fixed layout reads phi itself
  p.zero_offset = p.phip_offset + p.phip_bytes;
  p.rec_offset = p.zero_offset + 256;
  p.rec_bytes = pre ? (size_t)p.split * (size_t)B * (size_t)((n + 2) & ~1) * 4 : 0;
  p.flag_offset = p.rec_offset + ((p.rec_bytes + 15) & ~(size_t)15);
  p.total_bytes = p.flag_offset + (pre ? 16 : 0);
  return p;
}

int64_t pre_mode_grid(int64_t units, int64_t split, int64_t resident, int64_t wgs_cap) {
  if (units < 1 || split < 1 || resident < 1) return 0;
  int64_t cap = resident;
  if (wgs_cap >= 1 && wgs_cap < cap) cap = wgs_cap;
  cap = (cap / split) * split;  // whole row tiles per round
  if (cap < split) return 0;
  return units < cap ? units : cap;
}

namespace {
template <int MODE>
const void *pre_kernel_fn(int ni) {
  switch (ni) {
    case 0: return reinterpret_cast<const void *>(&post_res_next_kernel<1, MODE, true>);
    case 1: return reinterpret_cast<const void *>(&post_res_next_kernel<2, MODE, true>);
    default: return reinterpret_cast<const void *>(&post_res_next_kernel<4, MODE, true>);
  }
}
}  // namespace

int64_t pre_mode_resident(int n, int mode, hipStream_t st) {
  // Per-CU occupancy of the pre-mix kernel, cached per device and variant.
  static std::atomic<int> occ_cache[64][3][4];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int ni = n == 1 ? 0 : (n == 2 ? 1 : (n == 4 ? 2 : -1));
  const int mi = mode == kFusedApplyPreBf16 ? 0
               : mode == kFusedApplyPreFp8 ? 1
               : mode == kFusedCoeffsPreBf16 ? 2
               : mode == kFusedCoeffsPreFp8 ? 3 : -1;
  if (ni < 0 || mi < 0) return 0;
  int occ = (dev >= 0 && dev < 64) ? occ_cache[dev][ni][mi].load(std::memory_order_relaxed) : 0;
  if (occ <= 0) {
    const void *fn = mi == 0 ? pre_kernel_fn<kFusedApplyPreBf16>(ni)
                   : mi == 1 ? pre_kernel_fn<kFusedApplyPreFp8>(ni)
                   : mi == 2 ? pre_kernel_fn<kFusedCoeffsPreBf16>(ni)
                             : pre_kernel_fn<kFusedCoeffsPreFp8>(ni);
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, fn, FusedTile<4, true>::THREADS, 0) != hipSuccess) {
      (void)hipGetLastError();  // leave no sticky error for the launch check
      return 0;
    }
    occ = v;
    if (occ > 0 && dev >= 0 && dev < 64) occ_cache[dev][ni][mi].store(occ, std::memory_order_relaxed);
  }
  return (int64_t)occ * stream_cus(st);
}

int64_t stream_cus(hipStream_t st) {
  int64_t cus = device_cus();
  if (st != nullptr) {
    // A stream created with a CU mask runs on the masked CUs only.
    uint32_t mask[32] = {};
    const uint32_t words = (uint32_t)((cus + 31) / 32 <= 32 ? (cus + 31) / 32 : 32);
    if (hipExtStreamGetCUMask(st, words, mask) == hipSuccess) {
      int64_t on = 0;
      for (uint32_t w = 0; w < words; ++w) on += __builtin_popcount(mask[w]);
      if (on > 0 && on < cus) cus = on;
    } else {
      (void)hipGetLastError();
    }
  }
  return cus;
}

hipError_t launch_post_res_next(const FusedPlan &p, int n, int mode, int64_t B, int64_t C,
                                const void *X, const void *F, const float *H, void *Y,
                                const void *phi_next, void *ws_base, hipStream_t st,
                                const PreOut *pre_out) {
  const bool pre = is_pre_mode(mode);
  if (pre != p.pre || (pre && !pre_out)) return hipErrorInvalidValue;
  char *base = static_cast<char *>(ws_base);
  void *phip = base + p.phip_offset;
  // The fixed-slice layout gathers its phi operands from phi itself; the
  // other layouts read the packed copy.  The pre-mix mode's records and
  // give-up word start from zero.
  hipError_t e = hipSuccess;
  if (p.fixed)
    e = pre ? launch_zero(base + p.rec_offset, p.total_bytes - p.rec_offset, st) : hipSuccess;
  else
    e = launch_pack_phi(n, (int64_t)n * C, p.ksteps, phi_next, phip, base + p.zero_offset, st,
                        pre ? base + p.rec_offset : nullptr, p.total_bytes - p.rec_offset);
  if (e != hipSuccess) return e;
  float *ws = reinterpret_cast<float *>(base);
  float *dummy = reinterpret_cast<float *>(base + p.dummy_offset);
  const int spu = p.cw / kStepCh;
  const int64_t U = p.row_tiles * (int64_t)p.split;
  int cap = device_cus();
  PreArgs pa{};
  if (pre) {
    // Workgroups of one row tile wait for each other's records, so the whole
    // grid must be resident at once; the caller sized it (pre_mode_grid:
    // whole row tiles per round, within the resident count).
    const int64_t G = pre_out->grid;
    if (G < p.split || G % p.split != 0 || G > U) return hipErrorInvalidValue;
    cap = (int)G;
    pa.F_pre = pre_out->F_pre;
    pa.giveup = reinterpret_cast<uint32_t *>(base + p.flag_offset);
    pa.rec = reinterpret_cast<uint32_t *>(base + p.rec_offset);
    pa.rec_bytes = (uint32_t)p.rec_bytes;
    pa.partial_bytes = (uint32_t)p.partial_bytes;
    pa.b_pre = pre_out->b_pre;
    pa.alpha_pre = pre_out->alpha_pre;
    pa.inv_k = (float)(1.0 / (double)((int64_t)n * C));
  } else if (tune(kTuneFusedWgs) >= 1 && tune(kTuneFusedWgs) <= 65535) {
    cap = (int)tune(kTuneFusedWgs);
  }
  if (p.fixed) {
    // Whole row tiles per round (each workgroup keeps slice p(g) mod S).
    cap = (cap / p.split) * p.split;
    pa.phi = static_cast<const uint16_t *>(phi_next);
    pa.phi_bytes = (uint32_t)((int64_t)n * C * (n * n + 2 * n) * 2);
  }
  if (cap < 1) return hipErrorInvalidValue;
  const int G = (int)(U < cap ? U : cap);
  switch (mode) {
    case kFusedApplyBf16: return launch_mode<kFusedApplyBf16>(n, p.fixed, B, C, spu, p.split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case kFusedApplyFp8: return launch_mode<kFusedApplyFp8>(n, p.fixed, B, C, spu, p.split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case kFusedCoeffsFp8: return launch_mode<kFusedCoeffsFp8>(n, p.fixed, B, C, spu, p.split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case kFusedCoeffsBf16: return launch_mode<kFusedCoeffsBf16>(n, p.fixed, B, C, spu, p.split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case kFusedApplyPreBf16: return launch_mode<kFusedApplyPreBf16>(n, p.fixed, B, C, spu, p.split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case kFusedApplyPreFp8: return launch_mode<kFusedApplyPreFp8>(n, p.fixed, B, C, spu, p.split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case kFusedCoeffsPreBf16: return launch_mode<kFusedCoeffsPreBf16>(n, p.fixed, B, C, spu, p.split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    case kFusedCoeffsPreFp8: return launch_mode<kFusedCoeffsPreFp8>(n, p.fixed, B, C, spu, p.split, G, X, F, H, Y, phip, ws, dummy, pa, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mhc
