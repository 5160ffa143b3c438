// Split-K combine, coefficient gates and Sinkhorn-Knopp in one kernel.
//
// [mHC-cutile] (page "mHC 算法分析 & cutile 高效实现"):
//   section 2.2  r = sqrt(sum(X_t^2) / (n C)), no epsilon;
//   section 2.3  h = alpha * logit / r + b for the pre, post and res blocks;
//   section 2.4  H_pre = sigmoid(h), H_post = 2 sigmoid(h), H_res =
//                Sinkhorn-Knopp(exp(h)): 20 times, every row divided by its
//                sum, then every column by its sum;
//   sections 3.2, 3.3, 5.2, 5.3  these steps are tiny per row, so they are
//                fused after the split-K reduction in a single launch.
//
// Layout: a workgroup owns RB rows (RB = 256 / n, or 1 row when B is small);
// in phase 2, n consecutive lanes serve one row, lane i holding row i of that
// row's n x n res matrix.
//   phase 1  lanes sum the S partial slices [S, B, N+1] in a fixed order
//            (bitwise deterministic).  With RB = 256 / n the workgroup has
//            1024 lanes (16 waves: enough loads in flight per CU to stream
//            the partials), every lane owns one to three elements of the
//            block and adds all slices in order 0..S-1; for each slice the
//            workgroup's rows are one contiguous run, so the loads coalesce,
//            and all loads of a batch of slices are issued before they are
//            added.  With one row per workgroup (small B,
//            typically many slices) the 256 lanes form G = 256 / (N+1) groups;
//            group g adds slices g, g+G, g+2G, ... in order and the G group
//            sums are then added in group order.  Sums go to LDS and the raw
//            logits to global memory.
//            With TREE (at most 16 slices) the slices are instead added as
//            the balanced binary tree over 16 slots, zero past S
//            (tree16_sum_serial), the order in which the pre-mix mode of the
//            fused kernel sums the same partials for its H_pre; at n = 8 (at
//            most 32 slices) the trees of slots 0-15 and 16-31, then their
//            sum, the order of the n = 8 pass (mhc_onepass8.hip).
//   phase 2  finish_row (mhc_finish.h): lane i computes gate i of the pre
//            and post blocks, then the Sinkhorn iteration on row i of the res
//            matrix, with column sums by a DPP butterfly over the row's lanes.
#include "mhc_device.h"
#include "mhc_finish.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

constexpr int64_t kOneRowMaxB = 512;  // up to this many rows, one row per workgroup

constexpr int kMultiRowThreads = 1024;  // lanes per workgroup of the multi-row layout

template <int NS, bool ONE_ROW, bool TREE = false>
__global__ __launch_bounds__(ONE_ROW ? 256 : kMultiRowThreads) void coeff_sinkhorn_kernel(
    const float *__restrict__ ws, int split, int B, float inv_k, float alpha_pre,
    float alpha_post, float alpha_res, const float *__restrict__ b_pre,
    const float *__restrict__ b_post, const float *__restrict__ b_res,
    float *__restrict__ logits, float *__restrict__ r_out, float *__restrict__ H) {
  static_assert(NS == 1 || NS == 2 || NS == 4 || NS == 8, "n");
  constexpr int N = NS * NS + 2 * NS;
  constexpr int NP = N + 1;
  constexpr int R = ONE_ROW ? 1 : 256 / NS;  // rows per workgroup
  constexpr int G = ONE_ROW ? 256 / NP : 1;   // slice groups (one-row mode)
  __shared__ float sums[R * NP];
  __shared__ float gsum[ONE_ROW ? G * NP : 1];

  const int tid = threadIdx.x;
  const int row0 = blockIdx.x * R;
  const int rows = min(R, B - row0);

  if constexpr (ONE_ROW) {
    const size_t slice = (size_t)B * NP;
    const float *base = ws + (size_t)row0 * NP;
    const int g = tid / NP, e = tid - g * NP;
    if (g < G) {
      float acc = 0.f;
      for (int s0 = g; s0 < split; s0 += 4 * G) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (s0 + q * G < split) ? base[(size_t)(s0 + q * G) * slice + e] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (s0 + q * G < split) acc += v[q];
      }
      gsum[g * NP + e] = acc;
    }
    __syncthreads();
    if (tid < NP) {
      float a = 0.f;
#pragma unroll
      for (int q = 0; q < G; ++q) a += gsum[q * NP + tid];
      sums[tid] = a;
      if (tid < N) logits[(size_t)row0 * N + tid] = a;
    }
  } else {
    // Every thread owns EPT elements of the workgroup's [rows, N+1] block and
    // issues the loads of SB slices for all of them before adding, so a
    // thread has up to SB*EPT independent loads in flight.
    constexpr int TH = kMultiRowThreads;
    constexpr int EPT = (R * NP + TH - 1) / TH;
    constexpr int SB = 4;
    const size_t slice = (size_t)B * NP;
    const float *base = ws + (size_t)row0 * NP;
    const int nel = rows * NP;
    float acc[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) acc[q] = 0.f;
    if constexpr (TREE) {
      // Slots past S are zero (no load); the tree is the same for any S.  At
      // n = 8 there are 32 slots: the 16-slot trees of slots 0-15 and 16-31,
      // then their sum.
      constexpr int TS = NS >= 8 ? 32 : 16;
#pragma unroll
      for (int q = 0; q < EPT; ++q) {
        const int e = tid + q * TH;
        float part[TS / 16];
#pragma unroll
        for (int h = 0; h < TS / 16; ++h) {
          float v[16];
#pragma unroll
          for (int sb = 0; sb < 16; ++sb) v[sb] = 0.f;
          // Streaming loads: the partials are read once.  With plain loads
          // the one-pass call measured 400-403 against 394-395 us at
          // n=4, C=7168, B=16384 (the combine is its last launch).
          if (e < nel) {
#pragma unroll
            for (int sb = 0; sb < 16; ++sb)
              if (16 * h + sb < split) v[sb] = __builtin_nontemporal_load(base + (size_t)(16 * h + sb) * slice + e);
          }
          part[h] = tree16_sum_serial(v);
        }
        if constexpr (TS == 32)
          acc[q] = part[0] + part[1];
        else
          acc[q] = part[0];
      }
    }
    for (int s0 = 0; s0 < (TREE ? 0 : split); s0 += SB) {
      float v[SB][EPT];
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
          const int e = tid + q * TH;
          v[sb][q] = (s0 + sb < split && e < nel) ? base[(size_t)(s0 + sb) * slice + e] : 0.f;
        }
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int q = 0; q < EPT; ++q)
          if (s0 + sb < split) acc[q] += v[sb][q];
    }
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = tid + q * TH;
      if (e < nel) {
        sums[e] = acc[q];
        const int rr = e / NP, cc = e - rr * NP;
        if (cc < N) logits[(size_t)(row0 + rr) * N + cc] = acc[q];
      }
    }
  }
  __syncthreads();

  const int lr = tid / NS, i = tid % NS;
  if (lr >= rows) return;  // whole row groups leave together
  finish_row<NS>(sums + lr * NP, row0 + lr, i, inv_k, alpha_pre, alpha_post, alpha_res, b_pre,
                 b_post, b_res, r_out, H);
}

template <int NS>
void launch_n(int64_t B, int64_t C, int split, const float *ws, float ap, float aq, float ar,
              const float *bp, const float *bq, const float *br, float *logits, float *r,
              float *H, hipStream_t st, bool tree) {
  const float inv_k = (float)(1.0 / (double)(NS * C));
  if (tree) {
    constexpr int R = 256 / NS;
    coeff_sinkhorn_kernel<NS, false, true><<<dim3((uint32_t)((B + R - 1) / R)), kMultiRowThreads, 0, st>>>(
        ws, split, (int)B, inv_k, ap, aq, ar, bp, bq, br, logits, r, H);
    return;
  }
  // Small B: one row per workgroup, so that the slices are summed by many
  // lanes and many workgroups at once.
  if (B <= kOneRowMaxB) {
    coeff_sinkhorn_kernel<NS, true><<<dim3((uint32_t)B), 256, 0, st>>>(
        ws, split, (int)B, inv_k, ap, aq, ar, bp, bq, br, logits, r, H);
  } else {
    constexpr int R = 256 / NS;
    coeff_sinkhorn_kernel<NS, false><<<dim3((uint32_t)((B + R - 1) / R)), kMultiRowThreads, 0, st>>>(
        ws, split, (int)B, inv_k, ap, aq, ar, bp, bq, br, logits, r, H);
  }
}

}  // namespace

hipError_t launch_coeff_sinkhorn(int n, int64_t B, int64_t C, int split, const float *ws,
                                 float alpha_pre, float alpha_post, float alpha_res,
                                 const float *b_pre, const float *b_post, const float *b_res,
                                 float *logits, float *r, float *H, hipStream_t st, bool tree) {
  if (tree && split > (n == 8 ? kMaxSlices8 : 16)) return hipErrorInvalidValue;
  switch (n) {
    case 1: launch_n<1>(B, C, split, ws, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, st, tree); break;
    case 2: launch_n<2>(B, C, split, ws, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, st, tree); break;
    case 4: launch_n<4>(B, C, split, ws, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, st, tree); break;
    case 8: launch_n<8>(B, C, split, ws, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, st, tree); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mhc
