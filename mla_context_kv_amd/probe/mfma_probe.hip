// dcp_probe_mfma: a plain stream of v_mfma_f32_32x32x16_bf16 -- the matrix
// instruction of the stripe kernel -- on every SIMD, the measured bf16 MFMA
// peak that an MFMA-bound launch (Long verify) is also reported against.  A
// measurement tool in its own library (libdcp_probe.so), not part of the
// attention path.
//
// Each workgroup has 8 wavefronts (two per SIMD, as in the stripe kernel).
// A wave runs `iters` rounds of kChains independent accumulator chains, so
// the matrix core of its SIMD never waits on a result; operands stay in
// registers (no memory traffic) and hold hashed, data-like bit patterns.
// Every wave folds its accumulators into one float per lane of `sink`, so no
// MFMA is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWaves = 8;
constexpr int kChains = 4;
constexpr int64_t kFlopPerMfma = 32LL * 32 * 16 * 2;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// operand values: a hash of (lane, index, salt) mapped to about +-0.02, so the
// multiplier inputs toggle like real bf16 data (constant or zero operands
// draw less power and would flatter the peak)
__device__ __forceinline__ __bf16 operand(uint32_t lane, uint32_t i, uint32_t salt) {
  uint32_t x = lane * 0x9E3779B1u ^ (i + 1) * 0x85EBCA77u ^ salt * 0xC2B2AE3Du;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 13;
  return (__bf16)(((float)(x & 0xffff) - 32768.0f) * (0.02f / 32768.0f));
}

__global__ void __launch_bounds__(64 * kWaves) mfma_kernel(int32_t iters, float* __restrict__ sink) {
  const uint32_t lane = threadIdx.x;
  // a different A operand per chain, two B operands taken in turn
  bf16x8 a[kChains], b[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) a[c][i] = operand(lane, i, c + 1);
    b[0][i] = operand(lane, i, 11);
    b[1][i] = operand(lane, i, 12);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  // two rounds per trip, so every operand choice is fixed at compile time
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c & 1], acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[(c + 1) & 1], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Threads per workgroup of the MFMA probe (the sink holds one float per thread).
int dcp_probe_mfma_block_threads(void) { return 64 * kWaves; }

// dcp_probe_mfma -- `grid` workgroups of 8 waves, each wave issuing iters x 4
// MFMAs of 32x32x16 bf16 (iters rounded up to even); sink [grid][512] device
// float.  *flops (host,
// nullable) = the launch's matrix FLOPs.  Returns 0, -1 on a bad argument
// (nothing enqueued), -3 when the launch fails.
int dcp_probe_mfma(int32_t grid, int32_t iters, float* sink, int64_t* flops, void* stream) {
  if (grid < 1 || iters < 1 || sink == nullptr) return -1;
  const int64_t rounds = ((int64_t)iters + 1) / 2 * 2;
  if (flops) *flops = (int64_t)grid * kWaves * rounds * kChains * kFlopPerMfma;
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(64 * kWaves), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
