// dcp_probe_stream: a plain streaming read of device memory, the measured
// HBM read peak that the stripe-attention kernel's roofline is also reported
// against.  It is a measurement tool built into its own library
// (libdcp_probe.so), not part of the attention path.
//
// Every mode reads whole 36,864-byte pieces (one 32-token tile of 576-dim
// bf16 latent rows) once; the remainder of `bytes` past the last whole piece
// is not read.  Workgroup w reads a contiguous run of pieces.
//  mode 0: 16-byte direct-to-LDS non-temporal loads (global_load_lds_dwordx4
//          ... nt, the stripe kernel's tile load) issued by ONE wave per
//          workgroup of 8 waves into a 4-stage LDS ring, two pieces in flight
//          while one is read back: the stripe kernel's loader with its
//          compute taken out.  One workgroup per compute unit (LDS bound).
//  mode 1: the same loads issued by four waves per workgroup.
//  mode 2: 16-byte non-temporal loads into registers (no LDS), eight in
//          flight per lane, grid of `grid` workgroups of 256 threads.
// Each mode folds what it read into one word per thread of `sink` (so no
// load is dead) and never reads outside [src, src + bytes).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kPiece = 36864;                  // bytes per piece (one tile)
constexpr int kLoadsPerPiece = kPiece / 1024;  // 36 wave-wide 16-byte loads
constexpr int kStages = 4;
constexpr int kWaves = 8;

__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t off, uint32_t lds_addr) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(bu), "{m0}"(lds_addr) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_then_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// pieces [t0, t0 + n) of workgroup `id` out of G, for `tiles` pieces in all
__device__ __forceinline__ void my_range(int64_t tiles, int id, int G, int64_t& t0, int64_t& n) {
  const int64_t per = tiles / G, extra = tiles % G;
  t0 = (int64_t)id * per + (id < extra ? id : extra);
  n = per + (id < extra ? 1 : 0);
}

template <int kLoaderWaves>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * kWaves, 64 * kWaves)))
stream_lds_kernel(const char* __restrict__ src, int64_t tiles, uint32_t* __restrict__ sink) {
  static_assert(kLoadsPerPiece % kLoaderWaves == 0, "loads split evenly over the loader waves");
  constexpr int kMy = kLoadsPerPiece / kLoaderWaves;   // loads per piece of one loader wave
  constexpr int kTwo = 2 * kMy < 63 ? 2 * kMy : 63;    // vmcnt range: a larger count waits a little more
  __shared__ __align__(16) char smem[kStages * kPiece];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int64_t t0, n;
  my_range(tiles, blockIdx.x, gridDim.x, t0, n);
  const bool loader = wave < kLoaderWaves;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int64_t t) {
    if (!loader || t >= n) return;
    const char* base = src + (t0 + t) * (int64_t)kPiece;
    const uint32_t stage = lds0 + (uint32_t)(t % kStages) * kPiece;
#pragma unroll
    for (int k = 0; k < kMy; ++k) {
      const int g = k * kLoaderWaves + wave;           // load g covers bytes [1024 g, 1024 g + 1024)
      dma16_sbase(base, (uint32_t)(g * 1024 + lane * 16), stage + (uint32_t)(g * 1024));
    }
  };
  for (int64_t t = 0; t < kStages - 1; ++t) issue(t);
  uint32_t acc = 0;
  for (int64_t it = 0; it < n; ++it) {
    // piece it has landed (the loads of the later pieces already issued,
    // at most kStages - 2 of them, may still be in flight)
    const int64_t later = n - 1 - it < kStages - 2 ? n - 1 - it : kStages - 2;
    if (later >= 2) wait_vm_then_barrier<kTwo>();
    else if (later == 1) wait_vm_then_barrier<kMy>();
    else wait_vm_then_barrier<0>();
    // every wave is done with piece it-1: its stage takes piece it+3
    issue(it + kStages - 1);
    // read back 16 bytes per lane of the landed piece
    const uint4 v = *reinterpret_cast<const uint4*>(smem + (it % kStages) * kPiece + (wave * 64 + lane) * 16);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ void __launch_bounds__(256) stream_reg_kernel(const char* __restrict__ src, int64_t tiles,
                                                          uint32_t* __restrict__ sink) {
  // 16-byte units of the whole pieces, eight per lane per round, grid-stride
  const int64_t units = tiles * (kPiece / 16);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < units; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < units; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Threads per workgroup of a mode (the sink holds one word per thread).
int dcp_probe_block_threads(int32_t mode) { return mode == 2 ? 256 : 64 * kWaves; }

// dcp_probe_stream -- read the whole 36,864-byte pieces of [src, src + bytes)
// once with `grid` workgroups (mode 0/1: at most one per compute unit makes
// sense, LDS-bound), folding the data into sink [grid][threads] (device
// uint32).  *bytes_read (host, nullable) = pieces * 36,864.  Returns 0, -1 on
// a bad argument (nothing enqueued), -3 when the launch fails.
int dcp_probe_stream(const void* src, int64_t bytes, int32_t mode, int32_t grid, uint32_t* sink,
                     int64_t* bytes_read, void* stream) {
  if (src == nullptr || sink == nullptr || bytes < 0 || grid < 1 || mode < 0 || mode > 2) return -1;
  const int64_t tiles = bytes / kPiece;
  if (bytes_read) *bytes_read = tiles * kPiece;
  if (tiles == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  const char* p = (const char*)src;
  if (mode == 0)
    hipLaunchKernelGGL(stream_lds_kernel<1>, dim3(grid), dim3(64 * kWaves), 0, s, p, tiles, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(stream_lds_kernel<4>, dim3(grid), dim3(64 * kWaves), 0, s, p, tiles, sink);
  else
    hipLaunchKernelGGL(stream_reg_kernel, dim3(grid), dim3(256), 0, s, p, tiles, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
