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

template <int NS>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (NS >= 2) x = dpp_add_xor1(x);
  if constexpr (NS >= 4) x = dpp_add_xor2(x);
  if constexpr (NS >= 8) x = dpp_add_half_mirror(x);
  return x;
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
  const float r = sqrtf(sm[N] * inv_k);
  const float inv_r = 1.0f / r;
  float *h = H + (size_t)row * N;
  if (i == 0) r_out[row] = r;
  {
    const float zp = alpha_pre * sm[i] * inv_r + b_pre[i];
    h[i] = 1.0f / (1.0f + __expf(-zp));
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
