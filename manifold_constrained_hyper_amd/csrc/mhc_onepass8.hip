// The per-layer pass at n = 8: post/res apply of one layer, coefficient
// product of the next, and the next layer's pre-mix, in one read of the
// residual stream.
//
// [mHC-cutile] (page "mHC 算法分析 & cutile 高效实现"): section 2.5 gives
// X_{t+1} = H_res X_t + H_post^T F_out and, for the next layer, F_pre =
// sum_i H_pre[i] X_{t+1}[i]; sections 2.1-2.4 give the next layer's logits
// X_{t+1} . phi_{t+1} (n^2 + 2n = 80 columns), r from the row's sum of
// squares, and the gates.  Sections 3.4 and 5.4 fuse the apply so that X is
// read once and X_{t+1} written once.
//
// Why a kernel of its own at n = 8.  The n <= 4 pass (mhc_post_res_fused.hip)
// gives each workgroup a 512-channel slice of all n streams and holds the
// slice's phi block in registers.  At n = 8 that block is 4096 k x 80
// columns (640 KiB), more than a CU's registers; streaming it from L2 for
// every 16-row tile moves five times the X bytes.  Here a slice is 128
// channels of all 8 streams: 1024 k, a phi block of 160 KiB, 44 VGPRs per
// lane over 15 waves, gathered once per run and kept for every row tile the
// workgroup visits (the fixed-slice layout).
//
// Work decomposition.  S = ceil(C / 128) slices per row (at most 32);
// a persistent grid of G workgroups of 16 waves each, G a multiple of S
// (with the hand-off below all resident at once: the host sizes G from the
// occupancy the runtime reports and the stream's CUs).  Workgroup p (dealt so that each XCD takes a contiguous
// run of p, i.e. whole row tiles) keeps slice p mod S and visits row tiles
// p / S, p / S + G/S, ...  A step is one 16-row tile of its slice:
//   apply    wave w owns tile row w; lane l owns channels c0 + 2l, c0 + 2l + 1
//            of all 8 streams (one 4-byte word per stream: 256 contiguous
//            bytes per wave instruction).  X_{t+1} is post_res_kernel's
//            arithmetic (fp32 FMA chain from H_post * F_out, one
//            round-to-nearest-even), so it is bitwise mhc_post_res's; it goes
//            to HBM and, as bf16, into an LDS tile [16 rows][8][128]
//            (16-byte pieces XOR-swizzled by row);
//   product  15 waves = 5 column blocks x 3 k-groups of the tile's 32
//            32-channel k-steps (11, 11, 10): each reads its A operands from
//            the tile and multiplies them into its column block with
//            v_mfma_f32_16x16x32_bf16; the column-block-0 wave of each group
//            also forms the Gram block A A^T of its k-steps, whose diagonal
//            is the rows' sum of squares over them;
//   flush    in the next step, after its apply, the three k-group sums of
//            each (row, column) are added in k-group order (deterministic)
//            and stored as the slice's partials fp32 [S, B, 81]; the combine
//            kernel (coeff_sinkhorn_kernel, 32-slot tree order) turns them
//            into the next layer's logits, r and H.
// Each wave keeps the loads of the next two steps in flight (two register
// sets; one with the hand-off, whose records and gates leave no room for a
// second beside phi), and the step applies first so that the refill of its
// set is issued early.  Three LDS tiles: a step's rows stay until step t+3.
// Pre-mix (PRE): the flush also publishes, per (row, slice), the 8 pre
// logits and the sum of squares as 4-byte records [B][9][S] (zero until
// written, never zero when written: +0.0 is stored as -0.0; buffer stores
// with the SC1 bit, agent-scope coherent).  Two steps later each wave reads
// its row's 9 x S records, sums every column over the 32 slice slots as a
// balanced binary tree (zeros past S; the combine kernel's order, so H_pre
// comes out bitwise as in H_next), forms the 8 gates and emits the row's
// 128 channels of F_pre from the tile it kept (pre_kernel's arithmetic).
// Waits need only records published a step earlier by workgroups of the same
// round, and every workgroup publishes before it waits, so with the whole
// grid resident every wait ends; one that still cannot (kernels on other
// streams holding CUs) gives up after about a second, writes NaN to its F_pre
// and sets the give-up word (mhc_post_res_coeffs_pre_check reads it).
//
// Without APPLY the tile takes X itself (the first layer: mhc_coeffs_pre and
// mhc_coeffs at n = 8); without PRE no records and no F_pre.  Routes: the
// apply without the hand-off is mhc_post_res_coeffs at n = 8 (C <= 4096);
// the hand-off (one pass for mhc_post_res_coeffs_pre / mhc_coeffs_pre) and
// the product alone run only on request (MHC_PASS8_PRE, MHC_GEMM_ALGO=3):
// measured slower than the calls they replace at n=8, C=4096, B=8192.
#include "mhc_device.h"
#include "mhc_finish.h"
#include "mhc_launch.h"

#include <atomic>
#include <type_traits>

namespace mhc {

namespace {

constexpr int kNs = 8;
constexpr int kN = kNs * kNs + 2 * kNs;  // 80 logit columns
constexpr int kNP = kN + 1;              // ... and the sum of squares
constexpr int kSliceCh = 128;            // channels per slice (of every stream)
constexpr int kKs = kNs * kSliceCh / 32;  // 32-channel MFMA k-steps per slice: 32
constexpr int kR = 16;                    // rows per tile = waves per workgroup
constexpr int kThreads = 64 * kR;
constexpr int kRowBytes = kNs * kSliceCh * 2;  // one tile row: 2 KiB
constexpr int kTileBytes = kR * kRowBytes;     // 32 KiB
constexpr int kKg = 3;                         // k-groups of the product
constexpr int kKpg = (kKs + kKg - 1) / kKg;    // k-steps per group: 11 (the last has 10)
constexpr int kBlk = kN / 16;                  // column blocks: 5
constexpr int kGramWave = kKg * kBlk;          // waves of the product (wave 15 has none)
constexpr int kRedFloats = kKg * kR * kN;      // [k-group][row][column]
constexpr int kTiles = 3;                      // step t's rows stay until step t+3
constexpr int kLdsBytes = kTiles * kTileBytes + (kRedFloats + kKg * kR) * 4;
constexpr int kPreCols = kNs + 1;              // record columns: 8 pre logits, sum of squares
constexpr int kOuts = kR * kNP;                // flushed sums per step: 1296
constexpr int kOpt = (kOuts + kThreads - 1) / kThreads;
static_assert(kGramWave == kR - 1, "15 product waves");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

constexpr uint32_t kRecNegZero = 0x80000000u;
constexpr uint32_t kNone = 0x80000000u;  // a buffer offset past every buffer: access dropped / reads zero
constexpr int kSpinLimit = 1 << 17;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kSc1 = 16;  // cache policy bit SC1 (agent scope)
constexpr int kNt = 2;    // cache policy bit NT (streamed once)

struct Args8 {
  const uint8_t *X;  // bf16 [B, 8, C]
  const uint8_t *F;  // bf16 [B, C] (APPLY)
  const float *H;    // fp32 [B, 80] (APPLY)
  uint8_t *Y;        // bf16 [B, 8, C] (APPLY)
  const uint16_t *phi;
  uint32_t phi_bytes;
  float *ws;  // partials [S, B, 81]
  uint32_t partial_bytes;
  uint32_t *rec;  // records [B, 9, S] (PRE)
  uint32_t rec_bytes;
  uint32_t *giveup;  // (PRE)
  uint8_t *F_pre;    // bf16 [B, C] (PRE)
  const float *b_pre;
  float alpha_pre, inv_k;
  int B, C, S, row_tiles;
};

// SETS: register sets of loads in flight per wave (two do not fit the
// registers beside the pre-mix mode's).
template <bool APPLY, bool PRE, int SETS = PRE ? 1 : 2>
__global__ __launch_bounds__(kThreads) void onepass8_kernel(const Args8 a) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  float *red = reinterpret_cast<float *>(lds + kTiles * kTileBytes);
  float *gram_sm = red + kRedFloats;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int B = a.B, C = a.C, S = a.S;

  const int G = gridDim.x, gi = blockIdx.x;
  const int pg = (gi & 7) * (G >> 3) + min(gi & 7, G & 7) + (gi >> 3);
  const int slot = uniform(pg % S), tile0 = uniform(pg / S), gs = uniform(G / S);
  if (tile0 >= a.row_tiles) return;
  const int nsteps = (a.row_tiles - tile0 + gs - 1) / gs;
  const int c0 = slot * kSliceCh;
  const int c_end = min(C, c0 + kSliceCh);
  auto row0_of = [&](int t) { return uniform((tile0 + t * gs) * kR); };

  // This lane's two channels; lanes past the slice take the last pair in
  // range (they compute the owning lane's values, so their duplicate stores
  // rewrite identical bytes) and put zeros into the tile.
  const int cl = c0 + 2 * lane;
  const bool in_range = cl < c_end;
  const int cc = min(cl, c_end - 2);
  // 4-byte word of this lane in a tile row of stream i: piece (lane / 4) of
  // the stream's 16 pieces, swizzled by the row.  F_pre is read back from
  // the word of channel cc, so lanes past the slice store the owning lane's
  // bytes (their own words hold zeros).
  const int wofs = (((lane >> 2) ^ wave) << 4) + ((lane & 3) << 2);
  const int wofs_cc = ((((cc - c0) >> 3) ^ wave) << 4) + ((((cc - c0) >> 1) & 3) << 2);

  __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.ws, (short)0, (int)a.partial_bytes, kRsrcWord3);
  [[maybe_unused]] __amdgpu_buffer_rsrc_t rec_rsrc;
  if constexpr (PRE) rec_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.rec, (short)0, (int)a.rec_bytes, kRsrcWord3);

  // ---- phi operands of this wave, gathered once.  Wave (block nb, group kg)
  // holds, for each k-step ks of its group, lane (m, g) =
  // phi[k(ks) + 8g + j][16 nb + m], j = 0..7 (the B operand of
  // v_mfma_f32_16x16x32_bf16), where k(ks) is channel 32 (ks mod 4) of the
  // slice in stream ks / 4.  Steps past C are clamped into range; the tile is
  // zero there, so they add nothing.
  const int nb = wave % kBlk, kg = wave / kBlk;
  bf16x8 bfix[kKpg];
  {
    const __amdgpu_buffer_rsrc_t phi_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.phi), (short)0, (int)a.phi_bytes, kRsrcWord3);
#pragma unroll
    for (int q = 0; q < kKpg; ++q) {
      const int ks = kg * kKpg + q;
      const int i = ks >> 2, ts = ks & 3;
      const int kstep = (i * C + min(c0 + 32 * ts, C - 32)) >> 5;
      const bool used = wave < kGramWave && ks < kKs;
      const uint32_t base = used ? (uint32_t)((kstep * 32 + 8 * g) * kN + 16 * nb + m) * 2u : kNone;
      uint32_t w[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(phi_rsrc, base + (uint32_t)(2 * h * kN * 2), 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(phi_rsrc, base + (uint32_t)((2 * h + 1) * kN * 2), 0, 0);
        w[h] = lo | (hi << 16);
      }
      bfix[q] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    }
  }

  // ---- loads of one step: this wave's row of X (and F_out, H).  Rows past B
  // read row B-1 (their results are never stored, except the X_{t+1} words,
  // which are then row B-1's own bytes).
  struct Set {
    uint32_t x[kNs];
    uint32_t f;
    uint32_t h[2];
  };
  // Buffer accesses throughout: a row's resource in scalar registers, one
  // lane offset (cc * 2) for every stream, the stream in the scalar offset.
  const uint32_t voff = (uint32_t)cc * 2u;
  auto load_set = [&](Set &s, int t) {
    const int rr = uniform(min(row0_of(t) + wave, B - 1));
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.X) + (size_t)rr * kNs * C * 2, (short)0, kNs * C * 2, kRsrcWord3);
#pragma unroll
    for (int j = 0; j < kNs; ++j) s.x[j] = __builtin_amdgcn_raw_buffer_load_b32(xr, voff, j * C * 2, kNt);
    if constexpr (APPLY) {
      const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t *>(a.F) + (size_t)rr * C * 2, (short)0, C * 2, kRsrcWord3);
      s.f = __builtin_amdgcn_raw_buffer_load_b32(fr, voff, 0, kNt);
      // lane k holds H[row, 8 + k] (H_post, then H_res row-major), k < 72
      const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float *>(a.H) + (size_t)rr * kN, (short)0, kN * 4, kRsrcWord3);
      s.h[0] = __builtin_amdgcn_raw_buffer_load_b32(hrs, (uint32_t)(kNs + lane) * 4u, 0, 0);
      s.h[1] = __builtin_amdgcn_raw_buffer_load_b32(hrs, (uint32_t)(kNs + 64 + min(lane, 7)) * 4u, 0, 0);
    }
  };

  // ---- flush: the three k-group sums of step t's tile, in k-group order,
  // into its partials (and records).  Targets past B, and everything when
  // `real` is false, get an offset past the buffer (dropped).
  auto flush = [&](int t, bool real) {
    const int row0 = row0_of(t);
#pragma unroll
    for (int q = 0; q < kOpt; ++q) {
      const int e = tid + q * kThreads;
      const int ec = min(e, kOuts - 1);
      const int r = ec / kNP, col = ec - r * kNP;
      float v;
      if (col < kN)
        v = (red[r * kN + col] + red[(kR + r) * kN + col]) + red[(2 * kR + r) * kN + col];
      else
        v = (gram_sm[r] + gram_sm[kR + r]) + gram_sm[2 * kR + r];
      // partial (slot, row0 + r, col): the tile's rows are contiguous, so the
      // offset is e past the tile's first partial
      const bool tgt = real && e < kOuts && r < B - row0;
      const uint32_t poff = tgt ? (uint32_t)e * 4u : kNone;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ws_rsrc, poff, (slot * B + row0) * kNP * 4, 0);
      if constexpr (PRE) {
        const bool rec = tgt && (col < kNs || col == kN);
        const int rc = col < kNs ? col : kNs;
        const uint32_t roff = rec ? (uint32_t)((r * kPreCols + rc) * S) * 4u : kNone;
        const uint32_t bits = __float_as_uint(v);
        __builtin_amdgcn_raw_buffer_store_b32(bits == 0u ? kRecNegZero : bits, rec_rsrc, roff,
                                              (row0 * kPreCols * S + slot) * 4, kSc1);
      }
    }
  };

  // ---- records of step t's row of this wave: word (c, s) of the row in
  // load p, lane l: column c = 2p + l / 32, slot s = l mod 32 (zero past S or
  // past the 9 columns).
  typedef uint32_t rec_t[5];
  // The row's records start at scalar offset (rr * 9 + 2p) * S * 4 of load
  // p; a lane's offset past it selects its slot and column (lanes 32-63 of
  // load 4, which would be a tenth column, read nothing).
  const uint32_t rec_voff = (lane & 31) < S ? (uint32_t)((lane & 31) + (lane >> 5) * S) * 4u : kNone;
  const uint32_t rec_voff4 = lane < 32 ? rec_voff : kNone;
  auto rec_load = [&](rec_t &rv, int t) {
    const int rr = uniform(min(row0_of(t) + wave, B - 1));
#pragma unroll
    for (int p = 0; p < 5; ++p)
      rv[p] = __builtin_amdgcn_raw_buffer_load_b32(rec_rsrc, p < 4 ? rec_voff : rec_voff4,
                                                   (rr * kPreCols + 2 * p) * S * 4, kSc1);
  };
  auto rec_ready = [&](const rec_t &rv) -> bool {
    const int s = lane & 31;
    bool ok = true;
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      const int c = 2 * p + (lane >> 5);
      ok = ok && (!(c < kPreCols && s < S) || rv[p] != 0u);
    }
    return __builtin_amdgcn_ballot_w64(!ok) == 0;
  };
  auto rec_wait = [&](rec_t &rv, int t) -> bool {
    if (rec_ready(rv)) return false;
    bool ready = false;
    int tries = 0;
    do {
      __builtin_amdgcn_s_sleep(8);
      rec_load(rv, t);
      ready = rec_ready(rv);
    } while (!ready && ++tries < kSpinLimit);
    return !ready;
  };
  // H_pre of the row: each column summed over the 32 slots as the balanced
  // tree (16-slot trees, then the two halves added), every lane of a half
  // holding the sum; then gate i in lane i.
  [[maybe_unused]] float bpre_lane = 0.f;
  if constexpr (PRE) bpre_lane = a.b_pre[min(lane, kNs - 1)];
  auto pre_coeffs = [&](const rec_t &rv, float (&hp)[kNs]) {
    float t32[5];
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      const float t = tree16_sum(__uint_as_float(rv[p]));
      const float o = __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, __float_as_int(t)));
      t32[p] = t + o;  // (lower 16 slots) + (upper 16), the same bits in both halves
    }
    const float sq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t32[4]), 0));
    const float inv_r = recip_exact(row_rms(sq, a.inv_k));
    // lane i < 8 takes column i: t32[i / 2] from lane 32 (i mod 2)
    const int src = (lane & 1) << 7;
    float lg = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float v = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(t32[p])));
      lg = (lane >> 1) == p ? v : lg;
    }
    const float gate = pre_gate(lg, inv_r, a.alpha_pre, bpre_lane);
    // the gates broadcast in vector registers (scalar ones would not fit)
#pragma unroll
    for (int i = 0; i < kNs; ++i) hp[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(i << 2, __float_as_int(gate)));
  };
  // F_pre of this wave's row of step t from its tile (pre_kernel's chain:
  // from zero, stream order, one rounding).
  auto emit = [&](int t, int tile_idx, const float (&hp)[kNs], bool poison, bool real) {
    if (poison) {
      const __amdgpu_buffer_rsrc_t frs = __builtin_amdgcn_make_buffer_rsrc(a.giveup, (short)0, 4, kRsrcWord3);
      __builtin_amdgcn_raw_buffer_store_b32(1u, frs, 0u, 0, kSc1);
    }
    const int row = row0_of(t) + wave;
    const char *src = lds + tile_idx * kTileBytes + wave * kRowBytes + wofs_cc;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < kNs; ++j) {
      const uint32_t x = *reinterpret_cast<const uint32_t *>(src + j * (kSliceCh * 2));
      a0 = fmaf(hp[j], bf16_lo(x), a0);
      a1 = fmaf(hp[j], bf16_hi(x), a1);
    }
    uint32_t o = pack_bf16x2(a0, a1);
    if (poison) o = 0x7fc07fc0u;
    const bool tgt = real && row < B;
    const __amdgpu_buffer_rsrc_t frow = __builtin_amdgcn_make_buffer_rsrc(
        a.F_pre + (size_t)min(row, B - 1) * C * 2, (short)0, tgt ? C * 2 : 0, kRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b32(o, frow, voff, 0, 0);
  };

  // Step t uses tile t mod 3 (cur); the tile of step t-2 is (cur + 1) mod 3.
  auto step = [&](int t, int cur, Set &s, int t_pref) {
    // Order within the step: the apply first, so that the refill of this
    // register set is issued as early as possible; then the flush of step
    // t-1 and the F_pre of step t-2.
    [[maybe_unused]] rec_t rv;
    __syncthreads();  // red holds step t-1's sums; tile cur is free

    const int row0 = row0_of(t);
    const int rr = uniform(min(row0 + wave, B - 1));
    const bool live = row0 + wave < B;
    uint32_t out[kNs];
    if constexpr (APPLY) {
      const float f0 = bf16_lo(s.f), f1 = bf16_hi(s.f);
#pragma unroll
      for (int i = 0; i < kNs; ++i) {
        // the stream's nine coefficients are read from hv here, not all 72
        // at once (they would not fit the scalar registers)
        int h0 = (int)s.h[0], h1 = (int)s.h[1];
        asm volatile("" : "+v"(h0), "+v"(h1));
        const float hpost = __int_as_float(__builtin_amdgcn_readlane(h0, i));
        float a0 = hpost * f0, a1 = hpost * f1;
#pragma unroll
        for (int j = 0; j < kNs; ++j) {
          const int k = kNs + i * kNs + j;
          const float hr = __int_as_float(__builtin_amdgcn_readlane(k < 64 ? h0 : h1, k & 63));
          a0 = fmaf(hr, bf16_lo(s.x[j]), a0);
          a1 = fmaf(hr, bf16_hi(s.x[j]), a1);
        }
        out[i] = pack_bf16x2(a0, a1);
      }
      const __amdgpu_buffer_rsrc_t yr =
          __builtin_amdgcn_make_buffer_rsrc(a.Y + (size_t)rr * kNs * C * 2, (short)0, kNs * C * 2, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kNs; ++i) __builtin_amdgcn_raw_buffer_store_b32(out[i], yr, voff, i * C * 2, kNt);
    } else {
#pragma unroll
      for (int i = 0; i < kNs; ++i) out[i] = s.x[i];
    }
    char *trow = lds + cur * kTileBytes + wave * kRowBytes + wofs;
#pragma unroll
    for (int i = 0; i < kNs; ++i)
      *reinterpret_cast<uint32_t *>(trow + i * (kSliceCh * 2)) = (in_range && live) ? out[i] : 0u;
    load_set(s, t_pref);
    // (the records of step t-2 are read here, after the apply, whose
    // registers they would otherwise add to)
    if constexpr (PRE) rec_load(rv, t >= 2 ? t - 2 : 0);
    flush(t > 0 ? t - 1 : 0, t > 0);
    if constexpr (PRE) {
      // F_pre of step t-2 from this wave's row of its tile (its own row:
      // program order suffices; step t+1 rewrites that tile).
      const bool have = t >= 2;
      bool poison = false;
      if (have) poison = rec_wait(rv, t - 2);
      float hp[kNs];
      pre_coeffs(rv, hp);
      emit(have ? t - 2 : 0, cur == 2 ? 0 : cur + 1, hp, poison, have);
    }
    __syncthreads();  // the tile is complete; the flush has read red

    // product of tile cur
    const char *tile = lds + cur * kTileBytes;
    auto a_op = [&](int ks) {
      const int i = ks >> 2, ts = ks & 3;
      return *reinterpret_cast<const bf16x8 *>(tile + m * kRowBytes + i * (kSliceCh * 2) +
                                               ((((ts << 2) + g) ^ m) << 4));
    };
    // Every product wave runs its 11 k-steps without a branch (the tenth of
    // the last group is a copy of k-step 31 against zero phi), so the LDS
    // reads can run ahead of the MFMAs; the column-block-0 wave of each group
    // also forms the group's Gram block (the copy taken out by a zero A).
    auto product = [&](auto gram_tag) {
      constexpr bool GRAM = decltype(gram_tag)::value;
      // The A operand of k-step q+1 is read while q multiplies; the
      // scheduling barriers keep the compiler from reading further ahead
      // (which would cost registers the kernel does not have).
      f32x4 cv = {0.f, 0.f, 0.f, 0.f}, gv = {0.f, 0.f, 0.f, 0.f};
      bf16x8 an = a_op(kg * kKpg);
#pragma unroll
      for (int q = 0; q < kKpg; ++q) {
        const bf16x8 av = an;
        if (q + 1 < kKpg) an = a_op(min(kg * kKpg + q + 1, kKs - 1));
        cv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bfix[q], cv, 0, 0, 0);
        if constexpr (GRAM) {
          bf16x8 ag = av;
          if (q == kKpg - 1 && kg * kKpg + q >= kKs) ag = bf16x8{};
          gv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, ag, gv, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      float *rw = red + kg * kR * kN;
#pragma unroll
      for (int v = 0; v < 4; ++v) rw[(4 * g + v) * kN + 16 * nb + m] = cv[v];
      if constexpr (GRAM) {
        // diagonal (i, i) sits in lane i, register i & 3, of row group i / 4
        if (g == (m >> 2)) gram_sm[kg * kR + m] = gv[m & 3];
      }
    };
    if (wave < kGramWave) {
      if (nb == 0)
        product(std::true_type{});
      else
        product(std::false_type{});
    }
  };

  const int tl = nsteps - 1;
  if constexpr (SETS == 1) {
  // One register set: the loads of step t+1 are issued after step t's
  // apply.
  Set sa;
  load_set(sa, 0);
  int cur = 0;
  for (int t = 0; t < nsteps; ++t) {
    step(t, cur, sa, min(t + 1, tl));
    cur = cur == 2 ? 0 : cur + 1;
  }
  } else {
  // Two register sets: the loads of step t+2 are issued while step t runs.
  Set sa, sb;
  load_set(sa, 0);
  load_set(sb, min(1, tl));
  int t = 0, cur = 0;
  for (; t + 1 < nsteps; t += 2) {
    step(t, cur, sa, min(t + 2, tl));
    cur = cur == 2 ? 0 : cur + 1;
    step(t + 1, cur, sb, min(t + 3, tl));
    cur = cur == 2 ? 0 : cur + 1;
  }
  if (t < nsteps) step(t, cur, sa, tl);
  }
  __syncthreads();
  flush(tl, true);
  if constexpr (PRE) {
    // The last two steps' F_pre (their tiles are intact).
    auto tail = [&](int q) {
      rec_t rv;
      rec_load(rv, q);
      const bool poison = rec_wait(rv, q);
      float hp[kNs];
      pre_coeffs(rv, hp);
      emit(q, q % kTiles, hp, poison, true);
    };
    if (tl >= 1) tail(tl - 1);
    tail(tl);
  }
}

// Register sets of the hand-off variants (MHC_PASS8_SETS; default 1).
int pre_sets() { return tune(kTunePass8Sets) == 2 ? 2 : 1; }

template <bool APPLY, bool PRE>
const void *kernel_fn() {
  if (PRE && pre_sets() == 2) return reinterpret_cast<const void *>(&onepass8_kernel<APPLY, PRE, 2>);
  return reinterpret_cast<const void *>(&onepass8_kernel<APPLY, PRE>);
}

const void *kernel_of(bool apply, bool pre) {
  return apply ? (pre ? kernel_fn<true, true>() : kernel_fn<true, false>())
               : (pre ? kernel_fn<false, true>() : kernel_fn<false, false>());
}

}  // namespace

bool onepass8_fits(int64_t B, int64_t C) {
  if (B < 1 || C < 32 || C % 32 != 0) return false;
  const int64_t S = (C + kSliceCh - 1) / kSliceCh;
  const int64_t lim = int64_t(1) << 31;
  return S <= kMaxSlices8 && S <= device_cus() && (int64_t)kNs * C * kN * 2 < lim &&
         S * B * kNP * 4 < lim && B * kPreCols * S * 4 < lim && B * kNs * C * 2 < (int64_t(1) << 40);
}

FusedPlan plan_onepass8(int64_t B, int64_t C, bool pre) {
  FusedPlan p{};
  const int64_t S = (C + kSliceCh - 1) / kSliceCh;
  p.split = (int)S;
  p.cw = kSliceCh;
  p.row_tiles = (B + kR - 1) / kR;
  p.pre = pre;
  p.fixed = true;
  p.ksteps = (int64_t)kNs * C / 32;
  p.partial_bytes = (size_t)S * (size_t)B * kNP * sizeof(float);
  p.dummy_offset = (p.partial_bytes + 1023) & ~(size_t)1023;
  p.dummy_bytes = 0;
  p.phip_offset = p.dummy_offset;
  p.phip_bytes = 0;
  p.zero_offset = p.phip_offset;
  p.rec_offset = p.zero_offset;
  p.rec_bytes = pre ? (size_t)B * kPreCols * (size_t)S * 4 : 0;
  p.flag_offset = p.rec_offset + ((p.rec_bytes + 15) & ~(size_t)15);
  p.total_bytes = p.flag_offset + (pre ? 16 : 0);
  if (p.total_bytes < 16) p.total_bytes = 16;
  return p;
}

int64_t onepass8_resident(bool apply, bool pre, hipStream_t st) {
  static std::atomic<int> occ_cache[64][8];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const int vi = (apply ? 2 : 0) + (pre ? 1 : 0) + (pre && pre_sets() == 2 ? 4 : 0);
  int occ = (dev >= 0 && dev < 64) ? occ_cache[dev][vi].load(std::memory_order_relaxed) : 0;
  if (occ <= 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel_of(apply, pre), kThreads, 0) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    occ = v;
    if (occ > 0 && dev >= 0 && dev < 64) occ_cache[dev][vi].store(occ, std::memory_order_relaxed);
  }
  return (int64_t)occ * stream_cus(st);
}

hipError_t launch_onepass8(const FusedPlan &p, bool apply, int64_t B, int64_t C, const void *X,
                           const void *F, const float *H, void *Y, const void *phi, void *ws_base,
                           int64_t grid, hipStream_t st, const PreOut *pre_out) {
  const bool pre = p.pre;
  if (pre && !pre_out) return hipErrorInvalidValue;
  const int64_t U = p.row_tiles * (int64_t)p.split;
  if (grid < p.split || grid % p.split != 0 || grid > U) return hipErrorInvalidValue;
  char *base = static_cast<char *>(ws_base);
  if (pre) {
    // Records and the give-up word start from zero.
    const hipError_t e = launch_zero(base + p.rec_offset, p.total_bytes - p.rec_offset, st);
    if (e != hipSuccess) return e;
  }
  Args8 a{};
  a.X = static_cast<const uint8_t *>(X);
  a.F = static_cast<const uint8_t *>(F);
  a.H = H;
  a.Y = static_cast<uint8_t *>(Y);
  a.phi = static_cast<const uint16_t *>(phi);
  a.phi_bytes = (uint32_t)((int64_t)kNs * C * kN * 2);
  a.ws = reinterpret_cast<float *>(base);
  a.partial_bytes = (uint32_t)p.partial_bytes;
  a.B = (int)B;
  a.C = (int)C;
  a.S = p.split;
  a.row_tiles = (int)p.row_tiles;
  a.inv_k = (float)(1.0 / (double)(kNs * C));
  if (pre) {
    a.rec = reinterpret_cast<uint32_t *>(base + p.rec_offset);
    a.rec_bytes = (uint32_t)p.rec_bytes;
    a.giveup = reinterpret_cast<uint32_t *>(base + p.flag_offset);
    a.F_pre = static_cast<uint8_t *>(pre_out->F_pre);
    a.b_pre = pre_out->b_pre;
    a.alpha_pre = pre_out->alpha_pre;
  }
  const dim3 gr((uint32_t)grid), bl(kThreads);
  const bool two = pre_sets() == 2;
  if (apply) {
    if (pre && two) onepass8_kernel<true, true, 2><<<gr, bl, 0, st>>>(a);
    else if (pre) onepass8_kernel<true, true><<<gr, bl, 0, st>>>(a);
    else onepass8_kernel<true, false><<<gr, bl, 0, st>>>(a);
  } else {
    if (pre && two) onepass8_kernel<false, true, 2><<<gr, bl, 0, st>>>(a);
    else if (pre) onepass8_kernel<false, true><<<gr, bl, 0, st>>>(a);
    else onepass8_kernel<false, false><<<gr, bl, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mhc
