// Per-row finish of the coefficient computation, shared by the split-K combine
// kernel and the single-launch small-B kernel.
//
// [mHC-cutile] (page "mHC 算法分析 & cutile 高效实现"):
//   section 2.2  r = sqrt(sum(X_t^2) / (n C)), no epsilon;
//   section 2.3  h = alpha * logit / r + b for the pre, post and res blocks;
//   section 2.4  H_pre = sigmoid(h), H_post = 2 sigmoid(h), H_res =
//                Sinkhorn-Knopp(exp(h)): 20 times, every row divided by its
//                sum, then every column by its sum.
//
// n consecutive lanes serve one row; lane i computes gate i of the pre and
// post blocks and holds row i of the n x n res matrix.  A row normalisation
// is local to the lane; a column sum is a butterfly over the row's n lanes
// (DPP lane moves), after which every lane holds bitwise the same sum.
#pragma once

#include "mhc_device.h"

namespace mhc {

constexpr int kSinkhornIters = 20;

// x + (x from the lane whose index differs in the given low bits), for the
// butterfly over groups of 2, 4 or 8 aligned lanes.
__device__ __forceinline__ float dpp_add_xor1(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_add_xor2(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
// lane l <- lane (7 - l) within each group of 8: pairs the two quads of an
// aligned group of 8 once each quad holds its own sum.
__device__ __forceinline__ float dpp_add_half_mirror(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes as the balanced binary tree
// ((x0+x1)+(x2+x3)) + ... in slot order; every lane of the group ends with
// the same bits (each level adds two equal-shaped subtrees, and + commutes).
__device__ __forceinline__ float dpp_add_mirror(float x) {  // lane l <- lane 15 - l in its row of 16
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
}
__device__ __forceinline__ float tree16_sum(float x) {
  return dpp_add_mirror(dpp_add_half_mirror(dpp_add_xor2(dpp_add_xor1(x))));
}

// The same tree over 16 values held by one thread (slot order, zeros past the
// last slice): bitwise tree16_sum of those values.
__device__ __forceinline__ float tree16_sum_serial(const float (&x)[16]) {
  float y[8], z[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[2 * i] + x[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = y[2 * i] + y[2 * i + 1];
  return (z[0] + z[1]) + (z[2] + z[3]);
}

template <int NS>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (NS >= 2) x = dpp_add_xor1(x);
  if constexpr (NS >= 4) x = dpp_add_xor2(x);
  if constexpr (NS >= 8) x = dpp_add_half_mirror(x);
  return x;
}

// r of a row from its sum of squares (section 2.2, no epsilon) and 1/r.
__device__ __forceinline__ float row_rms(float sumsq, float inv_k) { return sqrtf(sumsq * inv_k); }
__device__ __forceinline__ float recip_exact(float r) { return 1.0f / r; }

// Gate i of the pre block (sections 2.3-2.4): sigmoid(alpha_pre * logit / r + b).
// Every kernel that forms H_pre calls this, so equal sums give equal bits.
__device__ __forceinline__ float pre_gate(float logit, float inv_r, float alpha_pre, float b) {
  const float z = alpha_pre * logit * inv_r + b;
  return 1.0f / (1.0f + __expf(-z));
}

// sm: the row's N+1 sums (N logits, then the sum of squares); lane i of the
// row's aligned group of n lanes.  Writes r[row] (lane 0) and H[row, :].
template <int NS>
__device__ __forceinline__ void finish_row(const float *sm, int row, int i, float inv_k,
                                           float alpha_pre, float alpha_post, float alpha_res,
                                           const float *__restrict__ b_pre,
                                           const float *__restrict__ b_post,
                                           const float *__restrict__ b_res,
                                           float *__restrict__ r_out, float *__restrict__ H) {
  constexpr int N = NS * NS + 2 * NS;
  const float r = row_rms(sm[N], inv_k);
  const float inv_r = recip_exact(r);
  float *h = H + (size_t)row * N;
  if (i == 0) r_out[row] = r;
  {
    h[i] = pre_gate(sm[i], inv_r, alpha_pre, b_pre[i]);
    const float zq = alpha_post * sm[NS + i] * inv_r + b_post[i];
    h[NS + i] = 2.0f / (1.0f + __expf(-zq));
  }

  float m[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j)
    m[j] = __expf(alpha_res * sm[2 * NS + i * NS + j] * inv_r + b_res[i * NS + j]);
  // Each normalisation multiplies by the hardware reciprocal of the sum
  // (v_rcp_f32, about 1 ulp) instead of dividing element by element.
#pragma unroll 1
  for (int it = 0; it < kSinkhornIters; ++it) {
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) rs += m[j];
    const float inv_rs = __builtin_amdgcn_rcpf(rs);
#pragma unroll
    for (int j = 0; j < NS; ++j) m[j] *= inv_rs;
#pragma unroll
    for (int j = 0; j < NS; ++j) m[j] *= __builtin_amdgcn_rcpf(group_sum<NS>(m[j]));
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) h[2 * NS + i * NS + j] = m[j];
}

}  // namespace mhc
