// Exact LSE merge kernel shared by dcp_lse_merge (merge across stripes) and
// the split-KV combine of dcp_stripe_attn (merge across the KV chunks of one
// stripe).  Both are the same operation: the softmax numerator and
// denominator are sums over a disjoint partition of the visible positions
// (page "DCP" (zdszero), "theory": merge identity, merge operator and
// numerical stability; the FlashAttention-style split inside a stripe is the
// same algebra on another axis, "unification with online softmax").
//
// With m = max_r lse_r: w_r = base^(lse_r - m), o = sum_r w_r o_r / sum_r w_r,
// lse = m + log_base(sum_r w_r).  Parts with lse = -inf have weight zero and
// their o is never read; if all parts are empty, o = 0 and lse = -inf.
//
// HBM-bound: per row it reads N lse values and N*v_dim floats once and
// writes v_dim + 1 floats.  One wavefront per row, 16-byte coalesced accesses.
#pragma once

#include "dcp_common.h"

namespace dcp {
namespace {   // internal linkage: each translation unit gets its own copy

constexpr int kMergeRowsPerBlock = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// part r of row i: o at o_parts[(r * rows + i) * v4 ...], lse at lse_parts[r * rows + i].
// in_base2 / out_base2 select the base of the input and output lse.
__global__ void __launch_bounds__(64 * kMergeRowsPerBlock)
lse_merge_kernel(int32_t N, int64_t rows, int32_t v4, const float4* __restrict__ o_parts,
                 const float* __restrict__ lse_parts, int32_t in_base2, int32_t out_base2,
                 float4* __restrict__ o, float* __restrict__ lse) {
  const int64_t r0 = (int64_t)blockIdx.x * kMergeRowsPerBlock + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (r0 >= rows) return;
  // weights are base^(lse_r - m): the difference is taken in the input base
  // (exact for nearby values) and only then scaled into base 2 for exp2
  const float to2 = in_base2 ? 1.0f : kLog2e;
  float m = -INFINITY;
  for (int r = 0; r < N; ++r) m = fmaxf(m, lse_parts[(int64_t)r * rows + r0]);
  if (m == -INFINITY) {
    for (int c = lane; c < v4; c += 64) o[r0 * v4 + c] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lse && lane == 0) lse[r0] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  for (int r = 0; r < N; ++r) {
    const float x = lse_parts[(int64_t)r * rows + r0];
    if (x == -INFINITY) continue;
    wsum += exp2f((x - m) * to2);
  }
  const float inv = 1.0f / wsum;
  for (int c = lane; c < v4; c += 64) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = 0; r < N; ++r) {
      const float x = lse_parts[(int64_t)r * rows + r0];
      if (x == -INFINITY) continue;
      const float w = exp2f((x - m) * to2) * inv;
      const float4 v = o_parts[((int64_t)r * rows + r0) * v4 + c];
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
    o[r0 * v4 + c] = acc;
  }
  if (lse && lane == 0) {
    // lse = m + log_base(sum w), written in the output base
    const float lw2 = log2f(wsum);                          // log2 of the weight sum
    const float m_out = (in_base2 == out_base2) ? m : (in_base2 ? m * kLn2 : m * kLog2e);
    lse[r0] = m_out + (out_base2 ? lw2 : lw2 * kLn2);
  }
}

inline int launch_lse_merge(int32_t N, int64_t rows, int32_t v_dim, const float* o_parts,
                            const float* lse_parts, int32_t in_base2, int32_t out_base2, float* o,
                            float* lse, hipStream_t stream) {
  const int64_t blocks = ceil_div(rows, kMergeRowsPerBlock);
  if (blocks > 0x7fffffff) return DCP_EUNSUPPORTED;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(64 * kMergeRowsPerBlock), 0,
                     stream, N, rows, v_dim / 4, (const float4*)o_parts, lse_parts, in_base2,
                     out_base2, (float4*)o, lse);
  return launch_status();
}

}  // namespace
}  // namespace dcp
