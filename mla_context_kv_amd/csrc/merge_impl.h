// Exact LSE merge kernel of dcp_lse_merge (merge across stripes), and the wave
// reductions and constants it shares with the split-KV combine of
// dcp_stripe_attn (merge across the KV chunks of one stripe, whose bf16 body
// sits beside the attention kernel).  Both are the same operation: the softmax numerator and
// denominator are sums over a disjoint partition of the visible positions
// (page "DCP" (zdszero), "theory": merge identity, merge operator and
// numerical stability; the FlashAttention-style split inside a stripe is the
// same algebra on another axis, "unification with online softmax").
//
// With m = max_r lse_r: w_r = base^(lse_r - m), o = sum_r w_r o_r / sum_r w_r,
// lse = m + log_base(sum_r w_r).  Parts with lse = -inf have weight zero and
// their o does not enter the result, whatever it holds (up to 8 parts it is
// read and selected away, above that it is not read); if all parts are
// empty, o = 0 and lse = -inf.
//
// HBM-bound: per row it reads N lse values and N*v_dim floats once and
// writes v_dim + 1 floats, with 16-byte coalesced accesses.
#pragma once

#include "dcp_common.h"

namespace dcp {
namespace {   // internal linkage: each translation unit gets its own copy

constexpr int kMergeRowsPerBlock = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Reductions over the wave's 64 lanes (every lane active), with a
// wave-uniform result: shifts of 1, 2, 4 and 8 lanes inside each row of 16
// leave each row's total in its lane 15, and the row broadcasts of lanes 15
// and 31 gather them in lane 63 -- cross-lane data paths of the VALU (DPP),
// where a shuffle through the LDS crossbar costs a round trip per step.  A
// lane with no source (past the row start, or a row the step leaves alone)
// reads the operation's identity.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_or(float identity, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), kCtrl,
                                                    kRowMask, 0xf, false));
}

__device__ __forceinline__ float wave_max(float v) {
  const float id = -INFINITY;
  v = fmaxf(v, dpp_or<0x111, 0xf>(id, v));   // row_shr:1
  v = fmaxf(v, dpp_or<0x112, 0xf>(id, v));   // row_shr:2
  v = fmaxf(v, dpp_or<0x114, 0xf>(id, v));   // row_shr:4
  v = fmaxf(v, dpp_or<0x118, 0xf>(id, v));   // row_shr:8
  v = fmaxf(v, dpp_or<0x142, 0xa>(id, v));   // row_bcast:15 into rows 1 and 3
  v = fmaxf(v, dpp_or<0x143, 0xc>(id, v));   // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_or<0x111, 0xf>(0.f, v);
  v += dpp_or<0x112, 0xf>(0.f, v);
  v += dpp_or<0x114, 0xf>(0.f, v);
  v += dpp_or<0x118, 0xf>(0.f, v);
  v += dpp_or<0x142, 0xa>(0.f, v);
  v += dpp_or<0x143, 0xc>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Where a merged row goes: its v4 16-byte column slices (c) and its lse.
// Fp32Out: o as float32 [v4 * 4] and lse as float32 (lse may be NULL).
struct Fp32Out {
  float4* __restrict__ o;
  float* __restrict__ l;
  __device__ void o4(int c, float4 v) const { o[c] = v; }
  __device__ bool has_lse() const { return l != nullptr; }
  __device__ void lse(float x) const { *l = x; }
};

// Merge of one row by one wavefront.  `src` gives part r's lse (src.lse(r))
// and its 16-byte column slice c as four floats (src.o4(r, c)); the result
// goes to o_row[0 .. v4) and *lse_out (when not NULL).  in_base2 / out_base2
// select the base of the input and output lse.  The lanes first hold the
// parts' lse (64 parts at a time) for the max and the weight sum, then every
// lane merges two 16-byte column slices, with the loads of 8 parts in flight
// before their FMAs.  Parts of weight zero (lse = -inf, or an underflowed
// weight) are never read.
template <class Src, class Dst>
__device__ __forceinline__ void merge_row(int32_t N, int32_t v4, const Src& src, int32_t in_base2,
                                          int32_t out_base2, const Dst& dst) {
  const int lane = threadIdx.x & 63;
  // weights are base^(lse_r - m): the difference is taken in the input base
  // (exact for nearby values) and only then scaled into base 2 for exp2
  const float to2 = in_base2 ? 1.0f : kLog2e;
  float m = -INFINITY;
  for (int r0 = 0; r0 < N; r0 += 64)
    if (r0 + lane < N) m = fmaxf(m, src.lse(r0 + lane));
  m = wave_max(m);
  if (m == -INFINITY) {
    for (int c = lane; c < v4; c += 64) dst.o4(c, make_float4(0.f, 0.f, 0.f, 0.f));
    if (dst.has_lse() && lane == 0) dst.lse(-INFINITY);
    return;
  }
  float wsum = 0.f;
  for (int r0 = 0; r0 < N; r0 += 64) {
    const float x = r0 + lane < N ? src.lse(r0 + lane) : -INFINITY;
    wsum += x == -INFINITY ? 0.f : exp2f((x - m) * to2);
  }
  wsum = wave_sum(wsum);
  const float inv = 1.0f / wsum;
  for (int cb = 0; cb < v4; cb += 128) {
    const int c0 = cb + lane, c1 = cb + 64 + lane;
    const bool in0 = c0 < v4, in1 = c1 < v4;
    float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
    for (int r0 = 0; r0 < N; r0 += 64) {
      const float x = r0 + lane < N ? src.lse(r0 + lane) : -INFINITY;
      const float w = x == -INFINITY ? 0.f : exp2f((x - m) * to2) * inv;   // lane k: weight of part r0 + k
      const int nr = min(64, N - r0);
      for (int u = 0; u < nr; u += 8) {
        float wu[8];
        float4 v0[8], v1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          wu[k] = u + k < nr ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u + k)) : 0.f;
          v0[k] = v1[k] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (wu[k] != 0.f) {
            if (in0) v0[k] = src.o4(r0 + u + k, c0);
            if (in1) v1[k] = src.o4(r0 + u + k, c1);
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          a0.x += wu[k] * v0[k].x;
          a0.y += wu[k] * v0[k].y;
          a0.z += wu[k] * v0[k].z;
          a0.w += wu[k] * v0[k].w;
          a1.x += wu[k] * v1[k].x;
          a1.y += wu[k] * v1[k].y;
          a1.z += wu[k] * v1[k].z;
          a1.w += wu[k] * v1[k].w;
        }
      }
    }
    if (in0) dst.o4(c0, a0);
    if (in1) dst.o4(c1, a1);
  }
  if (dst.has_lse() && lane == 0) {
    // lse = m + log_base(sum w), written in the output base
    const float lw2 = log2f(wsum);                          // log2 of the weight sum
    const float m_out = (in_base2 == out_base2) ? m : (in_base2 ? m * kLn2 : m * kLog2e);
    dst.lse(m_out + (out_base2 ? lw2 : lw2 * kLn2));
  }
}

// The same merge for at most kMax parts and v4 <= 128, with every load in
// flight at once: lane k < n holds part k's lse, and each lane loads its two
// 16-byte column slices of every part before the max is known.  One memory
// round trip instead of two.  A part of weight zero is read but selected
// away (never multiplied in), so whatever its buffer holds -- an empty
// stripe's unwritten output, NaN -- does not reach the result.
template <int kMax, class Src, class Dst>
__device__ __forceinline__ void merge_row_at_once(int32_t N, int32_t v4, const Src& src, int32_t in_base2,
                                                  int32_t out_base2, const Dst& dst) {
  const int lane = threadIdx.x & 63;
  const int c0 = lane, c1 = 64 + lane;
  const bool in0 = c0 < v4, in1 = c1 < v4;
  const float x = lane < N ? src.lse(lane) : -INFINITY;
  float4 a[kMax], b[kMax];
#pragma unroll
  for (int k = 0; k < kMax; ++k) {
    a[k] = b[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < N) {
      if (in0) a[k] = src.o4(k, c0);
      if (in1) b[k] = src.o4(k, c1);
    }
  }
  const float to2 = in_base2 ? 1.0f : kLog2e;
  const float m = wave_max(x);
  if (m == -INFINITY) {
    if (in0) dst.o4(c0, make_float4(0.f, 0.f, 0.f, 0.f));
    if (in1) dst.o4(c1, make_float4(0.f, 0.f, 0.f, 0.f));
    if (dst.has_lse() && lane == 0) dst.lse(-INFINITY);
    return;
  }
  const float e = x == -INFINITY ? 0.f : exp2f((x - m) * to2);
  const float wsum = wave_sum(e);
  const float w = e / wsum;
  float4 r0 = make_float4(0.f, 0.f, 0.f, 0.f), r1 = r0;
#pragma unroll
  for (int k = 0; k < kMax; ++k) {
    if (k < N) {
      const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
      if (wk != 0.f) {
        r0.x += wk * a[k].x; r0.y += wk * a[k].y; r0.z += wk * a[k].z; r0.w += wk * a[k].w;
        r1.x += wk * b[k].x; r1.y += wk * b[k].y; r1.z += wk * b[k].z; r1.w += wk * b[k].w;
      }
    }
  }
  if (in0) dst.o4(c0, r0);
  if (in1) dst.o4(c1, r1);
  if (dst.has_lse() && lane == 0) {
    const float lw2 = log2f(wsum);
    const float m_out = (in_base2 == out_base2) ? m : (in_base2 ? m * kLn2 : m * kLog2e);
    dst.lse(m_out + (out_base2 ? lw2 : lw2 * kLn2));
  }
}
constexpr int kAtOnceParts = 8;

// fp32 parts: part r of the row at o_parts[r * stride * v4 ...], lse at
// lse_parts[r * stride]
struct Fp32Parts {
  const float4* __restrict__ o;
  const float* __restrict__ l;
  int64_t stride;
  int32_t v4;
  __device__ float lse(int r) const { return l[(int64_t)r * stride]; }
  __device__ float4 o4(int r, int c) const { return o[(int64_t)r * stride * v4 + c]; }
};

__device__ __forceinline__ void merge_one_row(int32_t N, int64_t stride, int32_t v4,
                                              const float4* __restrict__ o_parts,
                                              const float* __restrict__ lse_parts, int32_t in_base2,
                                              int32_t out_base2, float4* __restrict__ o_row,
                                              float* __restrict__ lse_out) {
  const Fp32Parts src{o_parts, lse_parts, stride, v4};
  const Fp32Out dst{o_row, lse_out};
  if (N <= kAtOnceParts && v4 <= 128)
    merge_row_at_once<kAtOnceParts>(N, v4, src, in_base2, out_base2, dst);
  else
    merge_row(N, v4, src, in_base2, out_base2, dst);
}

// Part r of row i: o at o_parts[(r * rows + i) * v4 ...], lse at
// lse_parts[r * rows + i].  XCD-aware order: the dispatcher sends block i to
// XCD i % 8, so giving each XCD a contiguous range of rows keeps a request's
// rows on one XCD.
__global__ void __launch_bounds__(64 * kMergeRowsPerBlock)
lse_merge_kernel(int32_t N, int64_t rows, int32_t v4, const float4* __restrict__ o_parts,
                 const float* __restrict__ lse_parts, int32_t in_base2, int32_t out_base2,
                 float4* __restrict__ o, float* __restrict__ lse) {
  int64_t bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int64_t row = bid * kMergeRowsPerBlock + threadIdx.x / 64;
  if (row >= rows) return;
  merge_one_row(N, rows, v4, o_parts + row * v4, lse_parts + row, in_base2, out_base2, o + row * v4,
                lse ? lse + row : nullptr);
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
