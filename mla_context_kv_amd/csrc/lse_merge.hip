// dcp_lse_merge: exact merge of N stripes' partial results (the kernel and
// its derivation are in merge_impl.h).
#include "merge_impl.h"

extern "C" int dcp_lse_merge(int32_t n_stripes, int64_t rows, int32_t v_dim, const float* o_parts,
                             const float* lse_parts, int32_t lse_base, float* o, float* lse,
                             void* stream) {
  if (n_stripes < 1 || rows < 0 || v_dim <= 0 || v_dim % 4 != 0) return DCP_EINVAL;
  if (lse_base != 0 && lse_base != 1) return DCP_EINVAL;
  if (rows > 0 && (o_parts == nullptr || lse_parts == nullptr || o == nullptr)) return DCP_EINVAL;
  if (rows == 0) return DCP_OK;
  return dcp::launch_lse_merge(n_stripes, rows, v_dim, o_parts, lse_parts, lse_base, lse_base, o,
                               lse, (hipStream_t)stream);
}

// ---- the same merge over bf16 parts (o as bf16 beside a float32 lse, the
// partial payload of page "MLA 的 DCP", section 5).  One wavefront per output
// row; lane l takes values 8l .. 8l+7 (16 bytes of bf16) of each part, for
// column blocks of 512; the lse of up to 64 parts sit one per lane, and the
// loads of the first 8 parts go out with them (one memory round trip for up
// to 8 parts, one more per further 8).  The bf16 values widen exactly; every
// sum is float32.  Parts of weight zero are read but selected away.
namespace dcp {
namespace {

constexpr int kMergeBf16Waves = 4;     // output rows per block
constexpr int kMergeBf16Group = 8;     // parts in flight at once

__global__ void __launch_bounds__(64 * kMergeBf16Waves)
lse_merge_bf16_kernel(int32_t N, int64_t rows, int32_t v8, const uint4* __restrict__ o_parts,
                      const float* __restrict__ lse_parts, int32_t in_base2, int32_t out_base2,
                      float4* __restrict__ o, float* __restrict__ lse) {
  int64_t bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int lane = threadIdx.x & 63;
  const int64_t row = bid * kMergeBf16Waves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float to2 = in_base2 ? 1.0f : kLog2e;
  const float* const lse0 = lse_parts + row;
  const int64_t part_stride = rows * v8;          // uint4 units between parts
  float lp = lane < N ? lse0[(int64_t)lane * rows] : -INFINITY;
  float mx = lp;
  for (int r0 = 64; r0 < N; r0 += 64)
    if (r0 + lane < N) mx = fmaxf(mx, lse0[(int64_t)(r0 + lane) * rows]);
  for (int cb = 0; cb < v8; cb += 64) {
    const int c = cb + lane;
    const bool in = c < v8;
    const uint4* const part0 = o_parts + row * v8 + c;
    uint4 x[kMergeBf16Group];
#pragma unroll
    for (int k = 0; k < kMergeBf16Group; ++k)
      x[k] = k < N && in ? part0[k * part_stride] : make_uint4(0u, 0u, 0u, 0u);
    const float m = wave_max(mx);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lse_out = -INFINITY;
    if (m != -INFINITY) {
      float wsum = lp == -INFINITY ? 0.f : exp2f((lp - m) * to2);
      for (int r0 = 64; r0 < N; r0 += 64) {
        const float l = r0 + lane < N ? lse0[(int64_t)(r0 + lane) * rows] : -INFINITY;
        wsum += l == -INFINITY ? 0.f : exp2f((l - m) * to2);
      }
      wsum = wave_sum(wsum);
      const float inv = 1.0f / wsum;
      float w = lp == -INFINITY ? 0.f : exp2f((lp - m) * to2) * inv;   // lane k: weight of part r0 + k
      for (int g = 0; g < N; g += kMergeBf16Group) {
        if (g > 0) {
          if ((g & 63) == 0) {
            const float l = g + lane < N ? lse0[(int64_t)(g + lane) * rows] : -INFINITY;
            w = l == -INFINITY ? 0.f : exp2f((l - m) * to2) * inv;
          }
#pragma unroll
          for (int k = 0; k < kMergeBf16Group; ++k)
            x[k] = g + k < N && in ? part0[(g + k) * part_stride] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < kMergeBf16Group; ++k) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), (g + k) & 63));
          if (g + k < N && wk != 0.f) {
            const uint32_t u[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[2 * q] += wk * __uint_as_float(u[q] << 16);
              acc[2 * q + 1] += wk * __uint_as_float(u[q] & 0xffff0000u);
            }
          }
        }
      }
      const float lw2 = log2f(wsum);
      const float m_out = (in_base2 == out_base2) ? m : (in_base2 ? m * kLn2 : m * kLog2e);
      lse_out = m_out + (out_base2 ? lw2 : lw2 * kLn2);
    }
    if (in) {
      float4* const orow = o + row * (2 * (int64_t)v8);
      orow[2 * c] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      orow[2 * c + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    if (cb == 0 && lse != nullptr && lane == 0) lse[row] = lse_out;
  }
}

}  // namespace
}  // namespace dcp

extern "C" int dcp_lse_merge_bf16(int32_t n_parts, int64_t rows, int32_t v_dim, const void* o_parts,
                                  const float* lse_parts, int32_t lse_base, float* o, float* lse,
                                  void* stream) {
  if (n_parts < 1 || rows < 0 || v_dim <= 0 || v_dim % 8 != 0) return DCP_EINVAL;
  if (lse_base != 0 && lse_base != 1) return DCP_EINVAL;
  if (rows > 0 && (o_parts == nullptr || lse_parts == nullptr || o == nullptr)) return DCP_EINVAL;
  if (rows == 0) return DCP_OK;
  const int64_t blocks = dcp::ceil_div(rows, dcp::kMergeBf16Waves);
  // every part's row offsets (n_parts * rows * v_dim / 8 uint4 units) must fit 64 bits
  if (blocks > 0x7fffffff || rows > ((int64_t)1 << 62) / ((int64_t)n_parts * (v_dim / 8))) return DCP_EUNSUPPORTED;
  hipLaunchKernelGGL(dcp::lse_merge_bf16_kernel, dim3((unsigned)blocks), dim3(64 * dcp::kMergeBf16Waves), 0,
                     (hipStream_t)stream, n_parts, rows, v_dim / 8, (const uint4*)o_parts, lse_parts, lse_base,
                     lse_base, (float4*)o, lse);
  return dcp::launch_status();
}
