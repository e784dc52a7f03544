// Shared helpers of libdcp: layout arithmetic (host and device), argument
// checks and launch error handling.  Every function here is usable on both
// sides; nothing allocates.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcp.h"

#define DCP_HD __host__ __device__ __forceinline__

namespace dcp {

// Layout arithmetic for runs of I tokens handed out round robin to N ranks
// (page "PCP/DCP" (obnotes), section 6 "Block RR"; I = 1 is section 5).
struct Layout {
  int64_t N, I;
};

// owner(p) = floor(p / I) mod N
DCP_HD int64_t owner_of(const Layout& L, int64_t p) { return (p / L.I) % L.N; }

// row(p) = floor(p / (I*N)) * I + p mod I   (compact local row on the owner)
DCP_HD int64_t row_of(const Layout& L, int64_t p) { return (p / (L.I * L.N)) * L.I + p % L.I; }

// count_r(x): positions in [0, x) owned by rank r
//   = floor(x / (N*I)) * I + clamp(x mod (N*I) - r*I, 0, I)
DCP_HD int64_t count_of(const Layout& L, int64_t x, int64_t r) {
  if (x <= 0) return 0;
  const int64_t round = L.N * L.I;
  int64_t rem = x % round - r * L.I;
  rem = rem < 0 ? 0 : (rem > L.I ? L.I : rem);
  return (x / round) * L.I + rem;
}

// global position held by local row j of rank r
DCP_HD int64_t position_of(const Layout& L, int64_t j, int64_t r) {
  return (j / L.I) * L.I * L.N + r * L.I + j % L.I;
}

// host-side layout validation (the vLLM-Ascend CP design requires the page
// size to be a multiple of the interleave)
inline bool layout_ok(const dcp_layout& l) {
  return l.n_stripes >= 1 && l.interleave >= 1 && l.page_size >= 1 &&
         (l.page_size % l.interleave == 0 || l.interleave % l.page_size == 0);
}

inline Layout to_layout(const dcp_layout& l) { return Layout{l.n_stripes, l.interleave}; }

// Report DCP_ERANGE through the optional device status word (vector store).
__device__ __forceinline__ void flag_range(int32_t* status) {
  if (status) __hip_atomic_store(status, DCP_ERANGE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DCP_OK : DCP_EHIP;
}

// ceil(a / b) for a >= 0, b > 0, without forming a + b - 1 (no overflow near INT64_MAX)
inline int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0 ? 1 : 0); }

}  // namespace dcp
