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
// Layout: a workgroup of 256 lanes owns R = 256 / (n*n) rows.
//   phase 1  lanes sum the S partial slices [S, B, N+1] in slice order 0..S-1
//            (fixed order: bitwise deterministic).  For each slice the
//            workgroup's rows are one contiguous run, so the loads coalesce.
//            Sums go to LDS and the raw logits to global memory.
//   phase 2  each row is owned by n*n consecutive lanes; lane (i, j) holds
//            element (i, j) of the res matrix.  Row sums reduce over the low
//            log2(n) lane bits, column sums over the high bits, with xor
//            butterflies (every lane of a group ends with the same bits).
#include "mhc_device.h"
#include "mhc_launch.h"

namespace mhc {

namespace {

constexpr int kIters = 20;

template <int NS>
__global__ __launch_bounds__(256) void coeff_sinkhorn_kernel(
    const float *__restrict__ ws, int split, int B, float inv_k, float alpha_pre,
    float alpha_post, float alpha_res, const float *__restrict__ b_pre,
    const float *__restrict__ b_post, const float *__restrict__ b_res,
    float *__restrict__ logits, float *__restrict__ r_out, float *__restrict__ H) {
  constexpr int N = NS * NS + 2 * NS;
  constexpr int NP = N + 1;
  constexpr int L = NS * NS;   // lanes per row
  constexpr int R = 256 / L;   // rows per workgroup
  __shared__ float sums[R * NP];

  const int tid = threadIdx.x;
  const int row0 = blockIdx.x * R;
  const int rows = min(R, B - row0);

  {
    const size_t slice = (size_t)B * NP;
    const float *base = ws + (size_t)row0 * NP;
    for (int e = tid; e < rows * NP; e += 256) {
      // batches of 8 independent loads, added in slice order
      float a = 0.f;
      int s = 0;
      for (; s + 8 <= split; s += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = base[(size_t)(s + u) * slice + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) a += v[u];
      }
      for (; s < split; ++s) a += base[(size_t)s * slice + e];
      sums[e] = a;
      const int rr = e / NP, cc = e - rr * NP;
      if (cc < N) logits[(size_t)(row0 + rr) * N + cc] = a;
    }
  }
  __syncthreads();

  const int lr = tid / L, sub = tid - (tid / L) * L;
  if (lr >= rows) return;  // whole row groups leave together
  const float *sm = sums + lr * NP;
  const int row = row0 + lr;
  const float r = sqrtf(sm[N] * inv_k);
  const float inv_r = 1.0f / r;
  float *h = H + (size_t)row * N;
  if (sub == 0) r_out[row] = r;

  for (int c = sub; c < 2 * NS; c += L) {
    if (c < NS) {
      const float z = alpha_pre * sm[c] * inv_r + b_pre[c];
      h[c] = 1.0f / (1.0f + __expf(-z));
    } else {
      const float z = alpha_post * sm[c] * inv_r + b_post[c - NS];
      h[c] = 2.0f / (1.0f + __expf(-z));
    }
  }

  float v = __expf(alpha_res * sm[2 * NS + sub] * inv_r + b_res[sub]);
#pragma unroll 1
  for (int it = 0; it < kIters; ++it) {
    float rs = v;
#pragma unroll
    for (int o = 1; o < NS; o <<= 1) rs += __shfl_xor(rs, o, 64);
    v = v / rs;
    float cs = v;
#pragma unroll
    for (int o = NS; o < L; o <<= 1) cs += __shfl_xor(cs, o, 64);
    v = v / cs;
  }
  h[2 * NS + sub] = v;
}

template <int NS>
void launch_n(int64_t B, int64_t C, int split, const float *ws, float ap, float aq, float ar,
              const float *bp, const float *bq, const float *br, float *logits, float *r,
              float *H, hipStream_t st) {
  constexpr int R = 256 / (NS * NS);
  const dim3 grid((uint32_t)((B + R - 1) / R));
  const float inv_k = (float)(1.0 / (double)(NS * C));
  coeff_sinkhorn_kernel<NS><<<grid, 256, 0, st>>>(ws, split, (int)B, inv_k, ap, aq, ar, bp, bq,
                                                  br, logits, r, H);
}

}  // namespace

hipError_t launch_coeff_sinkhorn(int n, int64_t B, int64_t C, int split, const float *ws,
                                 float alpha_pre, float alpha_post, float alpha_res,
                                 const float *b_pre, const float *b_post, const float *b_res,
                                 float *logits, float *r, float *H, hipStream_t st) {
  switch (n) {
    case 1: launch_n<1>(B, C, split, ws, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, st); break;
    case 2: launch_n<2>(B, C, split, ws, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, st); break;
    case 4: launch_n<4>(B, C, split, ws, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, st); break;
    case 8: launch_n<8>(B, C, split, ws, alpha_pre, alpha_post, alpha_res, b_pre, b_post, b_res, logits, r, H, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mhc
