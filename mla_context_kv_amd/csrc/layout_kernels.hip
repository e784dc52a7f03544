// Integer side of DCP: slot map, per-rank interval counts, the
// owner-filtered paged KV write and the prefill-to-decode token relayout.
//
// Ownership is a pure function of the global position (page "DCP"
// (zdszero), "core abstraction", idea one); runs of I tokens go to the ranks
// in turn (page "PCP/DCP" (obnotes), section 6); a row's slot is its page id
// times the page size plus its offset in the page (page "PCP/DCP", "KV cache
// management"); a new latent row is stored only on its owner (page
// "MLA 的 Decode Context Parallelism", section 4, stage 2); a dense prefill
// cache is relaid out by selecting the positions a decode rank owns (page
// "PCP/DCP", "PD + DCP: extracting this rank's tokens from full source
// pages").
#include "dcp_common.h"

namespace dcp {
namespace {

constexpr int kThreads = 256;
constexpr int kLatentChunks = 576 * 2 / 16;   // 16-byte chunks of one latent row

int grid_for(int64_t work, int64_t per_block) {
  int64_t g = ceil_div(work, per_block);
  if (g < 1) g = 1;
  if (g > 16384) g = 16384;   // grid-stride loops cover the rest
  return static_cast<int>(g);
}

__global__ void __launch_bounds__(kThreads)
slot_map_kernel(Layout L, int64_t P, int32_t rank, const int64_t* __restrict__ pos,
                const int32_t* __restrict__ req, int64_t n, const int32_t* __restrict__ bt,
                int32_t bt_rows, int32_t bt_cols, int32_t* __restrict__ owner,
                int64_t* __restrict__ row, int64_t* __restrict__ slot, int32_t* status) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t p = pos[i];
    if (p < 0) {
      if (owner) owner[i] = -1;
      if (row) row[i] = -1;
      if (slot) slot[i] = -1;
      flag_range(status);
      continue;
    }
    const int64_t o = owner_of(L, p);
    const int64_t r = row_of(L, p);
    if (owner) owner[i] = (int32_t)o;
    if (row) row[i] = r;
    if (!slot) continue;
    int64_t s = -1;
    if (rank >= 0 && bt != nullptr && o == rank) {
      const int64_t b = req ? req[i] : 0;
      const int64_t col = r / P;
      if (b < 0 || b >= bt_rows || col >= bt_cols) {
        flag_range(status);
      } else {
        const int32_t pg = bt[b * bt_cols + col];
        if (pg < 0) flag_range(status);
        else s = (int64_t)pg * P + r % P;
      }
    }
    slot[i] = s;
  }
}

__global__ void __launch_bounds__(kThreads)
local_count_kernel(Layout L, const int64_t* __restrict__ start, const int64_t* __restrict__ len,
                   int64_t n, int64_t* __restrict__ count) {
  const int64_t total = n * L.N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total; k += stride) {
    const int64_t i = k / L.N;
    const int64_t r = k - i * L.N;
    const int64_t a = start ? start[i] : 0;
    const int64_t l = len[i];
    int64_t c = 0;
    if (a >= 0 && l > 0) c = count_of(L, a + l, r) - count_of(L, a, r);
    count[k] = c;
  }
}

// One new row per group of 8 lanes; each lane copies 16-byte chunks
// c, c+8, c+16, ... so a group moves 128 contiguous bytes per step.
__global__ void __launch_bounds__(kThreads)
kv_write_kernel(Layout L, int64_t P, int32_t rank, const uint4* __restrict__ kv_new,
                int32_t chunks, int64_t T, const int64_t* __restrict__ pos,
                const int32_t* __restrict__ req, const int32_t* __restrict__ bt,
                int32_t bt_rows, int32_t bt_cols, uint4* __restrict__ pool, int64_t num_pages,
                int32_t* status) {
  const int64_t groups = (int64_t)gridDim.x * (blockDim.x / 8);
  const int lane8 = threadIdx.x & 7;
  for (int64_t i = (int64_t)blockIdx.x * (blockDim.x / 8) + threadIdx.x / 8; i < T; i += groups) {
    const int64_t p = pos[i];
    if (p < 0) {
      if (lane8 == 0) flag_range(status);
      continue;
    }
    if (owner_of(L, p) != rank) continue;          // not ours: the row is not even read
    const int64_t r = row_of(L, p);
    const int64_t b = req ? req[i] : 0;
    const int64_t col = r / P;
    if (b < 0 || b >= bt_rows || col >= bt_cols) {
      if (lane8 == 0) flag_range(status);
      continue;
    }
    const int32_t pg = bt[b * bt_cols + col];
    if (pg < 0 || pg >= num_pages) {
      if (lane8 == 0) flag_range(status);
      continue;
    }
    const int64_t slot = (int64_t)pg * P + r % P;
    const uint4* src = kv_new + i * chunks;
    uint4* dst = pool + slot * chunks;
    for (int c = lane8; c < chunks; c += 8) dst[c] = src[c];
  }
}

// Prefill-to-decode token relayout: rank r's local rows j0 .. j1-1 of
// request b (j0 = count_r(start), j1 = count_r(start + len)) are the
// positions it owns in the chunk; row j holds position p = position_of(j),
// which sits at row p of the request's dense source pages.  One row per group
// of 8 lanes, 16-byte chunks as in the write above; grid y = request.
__global__ void __launch_bounds__(kThreads)
relayout_kernel(Layout L, int32_t rank, int32_t chunks, const uint4* __restrict__ src,
                int64_t src_pages, int64_t Ps, const int32_t* __restrict__ src_bt, int32_t src_cols,
                const int64_t* __restrict__ start, const int64_t* __restrict__ len,
                const int32_t* __restrict__ bt, int32_t bt_cols, int64_t Pd, uint4* __restrict__ dst,
                int64_t num_pages, int32_t* status) {
  const int64_t b = blockIdx.y;
  const int64_t a = start[b], l = len[b];
  const int lane8 = threadIdx.x & 7;
  if (a < 0 || l < 0) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag_range(status);
    return;
  }
  const int64_t j0 = count_of(L, a, rank), j1 = count_of(L, a + l, rank);
  const int64_t groups = (int64_t)gridDim.x * (blockDim.x / 8);
  for (int64_t j = j0 + (int64_t)blockIdx.x * (blockDim.x / 8) + threadIdx.x / 8; j < j1; j += groups) {
    const int64_t p = position_of(L, j, rank);
    const int64_t sc = p / Ps, dc = j / Pd;
    const int32_t spg = sc < src_cols ? src_bt[b * src_cols + sc] : -1;
    const int32_t dpg = dc < bt_cols ? bt[b * bt_cols + dc] : -1;
    if (spg < 0 || spg >= src_pages || dpg < 0 || dpg >= num_pages) {
      if (lane8 == 0) flag_range(status);
      continue;
    }
    const uint4* from = src + ((int64_t)spg * Ps + p % Ps) * chunks;
    uint4* to = dst + ((int64_t)dpg * Pd + j % Pd) * chunks;
    if (chunks == kLatentChunks) {
      // latent rows: all nine loads of the lane in flight before its stores
      uint4 v[kLatentChunks / 8];
#pragma unroll
      for (int k = 0; k < kLatentChunks / 8; ++k) v[k] = from[lane8 + 8 * k];
#pragma unroll
      for (int k = 0; k < kLatentChunks / 8; ++k) to[lane8 + 8 * k] = v[k];
    } else {
      for (int c = lane8; c < chunks; c += 8) to[c] = from[c];
    }
  }
}

// Sparse selection of one rank (page "DCP", conditions for merging: the
// top-k is chosen globally and each rank attends to the selected tokens it
// owns).  One workgroup per request walks its q_len * K selected positions in
// order and keeps those that are valid (0 <= p <= the draft's position) and
// owned by `rank`, with a workgroup prefix sum, so the list order is
// deterministic: entry = (local row, bit of the draft that selected it).
constexpr int kPlanThreads = 256;

__global__ void __launch_bounds__(kPlanThreads)
sparse_plan_kernel(Layout L, int32_t rank, int32_t q_len, int32_t K, const int32_t* __restrict__ topk,
                   const int32_t* __restrict__ seq_len, int32_t* __restrict__ rows, uint32_t* __restrict__ bits,
                   int32_t* __restrict__ count, int64_t stride) {
  __shared__ int32_t wave_tot[kPlanThreads / 64];
  const int64_t b = blockIdx.x;
  const int32_t S = seq_len[b];
  const int32_t n = q_len * K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* sel = topk + b * n;
  int32_t carry = 0;
  for (int32_t e0 = 0; e0 < n; e0 += kPlanThreads) {
    const int32_t e = e0 + threadIdx.x;
    bool keep = false;
    int64_t row = 0;
    uint32_t bit = 0;
    if (e < n) {
      const int32_t t = e / K;
      const int64_t pos = sel[e];
      if (pos >= 0 && pos <= (int64_t)S - q_len + t && owner_of(L, pos) == rank) {
        keep = true;
        row = row_of(L, pos);
        bit = 1u << t;
      }
    }
    const uint64_t mask = __builtin_amdgcn_ballot_w64(keep);
    const int32_t before_lane = __builtin_popcountll(mask & ((1ull << lane) - 1));
    if (lane == 0) wave_tot[wave] = __builtin_popcountll(mask);
    __syncthreads();
    int32_t before_wave = 0, total = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      before_wave += w < wave ? wave_tot[w] : 0;
      total += wave_tot[w];
    }
    if (keep) {
      const int64_t at = b * stride + carry + before_wave + before_lane;
      rows[at] = (int32_t)row;
      bits[at] = bit;
    }
    carry += total;
    __syncthreads();                                 // wave_tot is rewritten next round
  }
  if (threadIdx.x == 0) count[b] = carry;
}

}  // namespace
}  // namespace dcp

using namespace dcp;

extern "C" int dcp_slot_map(dcp_layout layout, int32_t rank, const int64_t* pos, const int32_t* req,
                            int64_t n, const int32_t* block_table, int32_t bt_rows, int32_t bt_cols,
                            int32_t* owner, int64_t* row, int64_t* slot, int32_t* status,
                            void* stream) {
  if (!layout_ok(layout) || n < 0) return DCP_EINVAL;
  if (rank < -1 || rank >= layout.n_stripes) return DCP_EINVAL;
  if (block_table && (bt_rows < 1 || bt_cols < 1)) return DCP_EINVAL;
  if (n > 0 && pos == nullptr) return DCP_EINVAL;
  if (n == 0) return DCP_OK;
  hipLaunchKernelGGL(slot_map_kernel, dim3(grid_for(n, kThreads)), dim3(kThreads), 0,
                     (hipStream_t)stream, to_layout(layout), (int64_t)layout.page_size, rank, pos,
                     req, n, block_table, bt_rows, bt_cols, owner, row, slot, status);
  return launch_status();
}

extern "C" int dcp_local_count(dcp_layout layout, const int64_t* start, const int64_t* len,
                               int64_t n, int64_t* count, void* stream) {
  if (!layout_ok(layout) || n < 0) return DCP_EINVAL;
  if (n > 0 && (len == nullptr || count == nullptr)) return DCP_EINVAL;
  if (n == 0) return DCP_OK;
  hipLaunchKernelGGL(local_count_kernel, dim3(grid_for(n * layout.n_stripes, kThreads)),
                     dim3(kThreads), 0, (hipStream_t)stream, to_layout(layout), start, len, n,
                     count);
  return launch_status();
}

extern "C" int dcp_kv_write(dcp_layout layout, int32_t rank, const void* kv_new, int32_t row_dim,
                            int64_t T, const int64_t* pos, const int32_t* req,
                            const int32_t* block_table, int32_t bt_rows, int32_t bt_cols,
                            void* pool, int64_t num_pages, int32_t* status, void* stream) {
  if (!layout_ok(layout) || T < 0) return DCP_EINVAL;
  if (rank < 0 || rank >= layout.n_stripes) return DCP_EINVAL;
  if (row_dim <= 0 || row_dim % 8 != 0) return DCP_EINVAL;
  if (block_table == nullptr || bt_rows < 1 || bt_cols < 1 || num_pages < 1 || pool == nullptr)
    return DCP_EINVAL;
  if (T > 0 && (kv_new == nullptr || pos == nullptr)) return DCP_EINVAL;
  if (T == 0) return DCP_OK;
  hipLaunchKernelGGL(kv_write_kernel, dim3(grid_for(T, kThreads / 8)), dim3(kThreads), 0,
                     (hipStream_t)stream, to_layout(layout), (int64_t)layout.page_size, rank,
                     (const uint4*)kv_new, row_dim / 8, T, pos, req, block_table, bt_rows, bt_cols,
                     (uint4*)pool, num_pages, status);
  return launch_status();
}

extern "C" int dcp_relayout(dcp_layout layout, int32_t rank, int32_t row_dim, const void* src_pool,
                            int64_t src_pages, int32_t src_page_size, const int32_t* src_block_table,
                            int32_t src_bt_cols, const int64_t* start, const int64_t* len, int32_t batch,
                            int64_t max_len, const int32_t* block_table, int32_t bt_cols, void* pool,
                            int64_t num_pages, int32_t* status, void* stream) {
  if (!layout_ok(layout) || rank < 0 || rank >= layout.n_stripes) return DCP_EINVAL;
  if (row_dim < 8 || row_dim % 8 != 0 || batch < 0 || max_len < 0) return DCP_EINVAL;
  if (src_page_size < 1 || src_pages < 1 || src_bt_cols < 1 || bt_cols < 1 || num_pages < 1) return DCP_EINVAL;
  if (batch == 0) return DCP_OK;
  if (batch > 65535) return DCP_EUNSUPPORTED;
  if (src_pool == nullptr || src_block_table == nullptr || len == nullptr || block_table == nullptr ||
      pool == nullptr || start == nullptr)
    return DCP_EINVAL;
  // rows of one request are at most its owned share of max_len positions
  const Layout L = to_layout(layout);
  const int64_t rows = (max_len / (L.N * L.I) + 1) * L.I;
  dim3 grid(grid_for(rows, kThreads / 8), (unsigned)batch);
  hipLaunchKernelGGL(relayout_kernel, grid, dim3(kThreads), 0, (hipStream_t)stream, L, rank, row_dim / 8,
                     (const uint4*)src_pool, src_pages, (int64_t)src_page_size, src_block_table, src_bt_cols,
                     start, len, block_table, bt_cols, (int64_t)layout.page_size, (uint4*)pool, num_pages, status);
  return launch_status();
}

extern "C" int dcp_sparse_plan(dcp_layout layout, int32_t rank, int32_t batch, int32_t q_len, int32_t topk,
                               const int32_t* topk_pos, const int32_t* seq_len, int32_t* rows, uint32_t* bits,
                               int32_t* count, int32_t stride, void* stream) {
  if (!layout_ok(layout) || rank < 0 || rank >= layout.n_stripes) return DCP_EINVAL;
  if (batch < 0 || q_len < 1 || topk < 1) return DCP_EINVAL;
  if (q_len > 32) return DCP_EUNSUPPORTED;
  if ((int64_t)q_len * topk > 0x7fffffff || stride < (int64_t)q_len * topk) return DCP_EINVAL;
  if (batch == 0) return DCP_OK;
  if (topk_pos == nullptr || seq_len == nullptr || rows == nullptr || bits == nullptr || count == nullptr)
    return DCP_EINVAL;
  hipLaunchKernelGGL(sparse_plan_kernel, dim3((unsigned)batch), dim3(kPlanThreads), 0, (hipStream_t)stream,
                     to_layout(layout), rank, q_len, topk, topk_pos, seq_len, rows, bits, count, (int64_t)stride);
  return launch_status();
}
