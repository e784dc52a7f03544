// Head-return exchange of DCP decode: the packed all-to-all payload and the
// owner's merge.
//
// Page "DCP" (zdszero), "merge: All-to-All": each rank cuts its partial
// output by head into N slices and sends slice d, with the matching LSE, in
// one packed buffer to the rank that owns those heads; the owner merges the N
// partials of its H/N heads with the exact LSE merge.  Page "MLA 的 Decode
// Context Parallelism", section 4: the payload is (512 + 4) 16-bit slots per
// (row, head) -- the output in bf16, then the LSE.  A record here is v_dim
// bf16 values, the float32 LSE in the next two slots and two zero slots, so
// records are 8-byte aligned (1032 bytes at v_dim = 512).
//
// Both kernels are HBM-bound: the pack reads 4 v_dim + 4 bytes and writes
// 2 v_dim + 8 bytes per (row, head); the merge reads N records per output row
// and writes v_dim + 1 floats.
#include "merge_impl.h"

namespace dcp {
namespace {

constexpr int kPackThreads = 256;

// float32 -> bfloat16, round to nearest even (the conversion instruction of
// gfx950 rounds this way)
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t h = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

// One thread per 4 output values of one (row, head); the thread of the first
// 4 also writes the record's LSE and padding.  Consecutive threads write
// consecutive 8-byte pieces of a record.
__global__ void __launch_bounds__(kPackThreads)
pack_heads_kernel(int32_t N, int64_t rows, int32_t H, int32_t v4, const float4* __restrict__ o_r,
                  const float* __restrict__ lse_r, uint2* __restrict__ send) {
  const int32_t Hl = H / N;
  const int64_t rec2 = v4 + 1;                         // record length in 8-byte units
  const int64_t total = rows * H * v4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t rh = t / v4;                         // row * H + h
    const int32_t c = (int32_t)(t - rh * v4);
    const int64_t row = rh / H;
    const int32_t h = (int32_t)(rh - row * H);
    const int32_t d = h / Hl, j = h - d * Hl;
    uint2* rec = send + (((int64_t)d * rows + row) * Hl + j) * rec2;
    const float4 x = o_r[t];
    rec[c] = make_uint2(pack2_bf16(x.x, x.y), pack2_bf16(x.z, x.w));
    if (c == 0) rec[v4] = make_uint2(__float_as_uint(lse_r[rh]), 0u);
  }
}

// part r of the owner's row i: record (r, i) of the received buffer
struct PackedParts {
  const uint2* __restrict__ recv;
  int64_t rows;
  int32_t v4;
  __device__ const uint2* rec(int r) const { return recv + ((int64_t)r * rows) * (v4 + 1); }
  __device__ float lse(int r) const { return __uint_as_float(rec(r)[v4].x); }
  __device__ float4 o4(int r, int c) const {
    const uint2 u = rec(r)[c];
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
};

__global__ void __launch_bounds__(64 * kMergeRowsPerBlock)
merge_heads_kernel(int32_t N, int64_t rows, int32_t v4, const uint2* __restrict__ recv, int32_t base2,
                   float4* __restrict__ o, float* __restrict__ lse) {
  int64_t bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int64_t row = bid * kMergeRowsPerBlock + threadIdx.x / 64;
  if (row >= rows) return;
  const PackedParts src{recv + row * (v4 + 1), rows, v4};
  const Fp32Out dst{o + row * v4, lse ? lse + row : nullptr};
  if (N <= kAtOnceParts && v4 <= 128)
    merge_row_at_once<kAtOnceParts>(N, v4, src, base2, base2, dst);
  else
    merge_row(N, v4, src, base2, base2, dst);
}

}  // namespace
}  // namespace dcp

using namespace dcp;

extern "C" int dcp_pack_heads(int32_t n_stripes, int64_t rows, int32_t n_heads, int32_t v_dim,
                              const float* o_r, const float* lse_r, void* send, void* stream) {
  if (n_stripes < 1 || rows < 0 || n_heads < 1 || n_heads % n_stripes != 0) return DCP_EINVAL;
  if (v_dim < 4 || v_dim % 4 != 0) return DCP_EINVAL;
  if (rows == 0) return DCP_OK;
  if (o_r == nullptr || lse_r == nullptr || send == nullptr) return DCP_EINVAL;
  if (rows > INT64_MAX / n_heads / (v_dim / 4)) return DCP_EUNSUPPORTED;   // (row, head, 4 values) count in 64 bits
  const int64_t total = rows * n_heads * (v_dim / 4);
  int64_t g = ceil_div(total, kPackThreads);
  g = g < 1 ? 1 : (g > 65536 ? 65536 : g);
  hipLaunchKernelGGL(pack_heads_kernel, dim3((unsigned)g), dim3(kPackThreads), 0, (hipStream_t)stream,
                     n_stripes, rows, n_heads, v_dim / 4, (const float4*)o_r, lse_r, (uint2*)send);
  return launch_status();
}

extern "C" int dcp_merge_heads(int32_t n_stripes, int64_t rows, int32_t v_dim, const void* recv,
                               int32_t lse_base, float* o, float* lse, void* stream) {
  if (n_stripes < 1 || rows < 0 || v_dim < 4 || v_dim % 4 != 0) return DCP_EINVAL;
  if (lse_base != 0 && lse_base != 1) return DCP_EINVAL;
  if (rows == 0) return DCP_OK;
  if (recv == nullptr || o == nullptr) return DCP_EINVAL;
  const int64_t blocks = ceil_div(rows, kMergeRowsPerBlock);
  if (blocks > 0x7fffffff) return DCP_EUNSUPPORTED;
  hipLaunchKernelGGL(merge_heads_kernel, dim3((unsigned)blocks), dim3(64 * kMergeRowsPerBlock), 0,
                     (hipStream_t)stream, n_stripes, rows, v_dim / 4, (const uint2*)recv, lse_base, (float4*)o, lse);
  return launch_status();
}
