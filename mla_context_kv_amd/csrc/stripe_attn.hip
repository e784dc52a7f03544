// dcp_stripe_attn: one rank's local attention of absorbed-MLA decode over its
// stripe of the latent KV, returning the locally normalised output o_r and
// its log-sum-exp lse_r.
//
// What is computed (page "MLA 的 Decode Context Parallelism", sections 2-3;
// page "DCP" (zdszero), idea two): every query row (request b, draft t,
// head h) is a 576-dim vector; each cached token is one shared 576-dim latent
// row whose whole row is the key and whose first 512 dims are the value.  The
// rank sees only the tokens it owns, stored compactly (local row j holds
// global position floor(j/I)*I*N + r*I + j mod I).  A query at global
// position S_b - q_len + t sees positions <= its own, i.e. the first
// count_r(S_b - q_len + t + 1) local rows (SGLang DCP docs, "DCP x
// speculative decoding": global lengths keep causality).
//
// How (MI355X / gfx950):
//  * One workgroup per (request, KV split, group of up to 128 query rows);
//    W = 1..4 wavefronts, each owning 32 query rows (heads are the N side of
//    the MFMA tiles, so the latent tile read from LDS serves all of them).
//  * KV tiles of 32 tokens are streamed HBM -> LDS with 16-byte direct-to-LDS
//    loads into a 3-4 stage ring; a tile's token rows are padded to 73
//    16-byte chunks so that both LDS access patterns below are bank-conflict
//    free.  The same LDS tile is the key (QK^T) and the value (PV): every KV
//    byte is read from HBM once.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (M = 32 tokens, N = 32 query
//    rows, K = 576 in 36 steps); Q stays in registers for the whole kernel.
//  * Online softmax in base 2 (scale * log2(e) folded in), row max over the
//    tile with one lane-half exchange; the reference max only moves when it
//    grows by more than 2^8, so the O rescale is rare and still exact.
//  * O^T += V^T P^T with the same MFMA (M = 32 value columns x 16 blocks,
//    N = 32 query rows, K = 16 tokens): P^T comes straight from the S^T
//    accumulator registers (no data movement), V^T is read from the
//    token-major LDS tile with ds_read_b64_tr_b16 transpose reads.
//  * Split-KV: when there are fewer (request, row group) items than compute
//    units, each request's stripe is cut into equal chunks of whole tiles; a
//    chunk writes its (o, lse) partial to the workspace and a second launch
//    merges the chunks with the same exact LSE merge as across stripes (the
//    chunks are a disjoint partition of the stripe's rows).
#include "dcp_common.h"
#include "merge_impl.h"

namespace dcp {
namespace attn {

constexpr int kD = 576;                 // latent row = key dims
constexpr int kDV = 512;                // value dims
constexpr int kChunks = kD / 8;         // 72 chunks of 16 bytes per row
constexpr int kTile = 32;               // tokens per tile
constexpr int kRowSlots = kChunks + 1;  // padded row: 73 chunks
constexpr int kTileSlots = kTile * kRowSlots;  // 2336
constexpr int kKSteps = kD / 16;        // 36 MFMA k-steps for QK^T
constexpr int kColBlocks = kDV / 32;    // 16 value-column blocks
constexpr int kRowBytes = kD * 2;       // 1152
// LDS operand prefetch depth (MFMA steps) of the QK^T and PV chains
#ifndef DCP_QK_AHEAD
#define DCP_QK_AHEAD 3
#endif
#ifndef DCP_PV_AHEAD
#define DCP_PV_AHEAD 3
#endif
constexpr int kQkAhead = DCP_QK_AHEAD;
constexpr int kPvAhead = DCP_PV_AHEAD;
static_assert(kQkAhead >= 1 && kQkAhead <= 15 && kPvAhead >= 1 && kPvAhead <= 7, "LDS counter range");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int W>
struct Shape {
  static constexpr int kThreads = 64 * W;
  static constexpr int kLoads = (kTileSlots + 64 * W - 1) / (64 * W);  // DMA loads / wave / tile
  static constexpr int kStageBytes = kLoads * 64 * W * 16;
  static constexpr int kStages = (W == 1) ? 3 : 4;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kWaitLoads = (kStages - 2) * kLoads;               // loads still in flight
  static_assert(kLdsBytes <= 163840, "LDS budget");
  static_assert(kWaitLoads <= 63, "vmcnt range");
};

// A zero latent row (plus pad chunk): what a tile slot holds when its page id
// is out of range (the call also flags DCP_ERANGE), so a bad table never
// makes the kernel read outside the pool.
__device__ __align__(16) uint4 g_zero_row[kRowSlots];

struct Params {
  int32_t N, I, P, rank;
  int32_t B, q_len, H, M;          // M = q_len * H query rows per request
  int32_t W, mgroups, splits, split_rows;
  const __bf16* q;
  const char* pool;
  int64_t num_pages;
  const int32_t* bt;
  int32_t bt_cols;
  const int32_t* seq_len;
  float c2;                         // scale * log2(e)
  int32_t out_base2;
  float* o;                         // final outputs (splits == 1)
  float* lse;
  float* ws_o;                      // split partials [splits][B][M][512], lse2 [splits][B][M]
  float* ws_lse;
  int32_t* status;
};

// 32-bit layout arithmetic (positions < 2^31: seq_len is int32)
__device__ __forceinline__ int32_t count_rows(int32_t x, int32_t N, int32_t I, int32_t r) {
  if (x <= 0) return 0;
  const int32_t round = N * I;
  int32_t rem = x % round - r * I;
  rem = rem < 0 ? 0 : (rem > I ? I : rem);
  return (x / round) * I + rem;
}

// MFMA row m of the QK^T A operand <-> token of the tile.  Within each group
// of 16, rows are transposed 4x4 so that a transpose read of V (4 tokens at
// once) touches 4 token rows 4 apart, which the 73-chunk row padding puts in
// disjoint LDS banks.
__device__ __forceinline__ int tau(int m) { return 16 * (m >> 4) + 4 * (m & 3) + ((m >> 2) & 3); }

__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_addr) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_then_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait until only the loads of the `after` most recent tiles (each kLoads
// per wave) are in flight, then barrier.  Tiles past the split issue no loads,
// so near the end fewer tiles are in flight and the count drops with them.
template <int kMaxAfter, int kLoads>
__device__ __forceinline__ void wait_tiles_then_barrier(int after) {
  static_assert(kMaxAfter == 1 || kMaxAfter == 2, "ring depth");
  if (after >= kMaxAfter) wait_vm_then_barrier<kMaxAfter * kLoads>();
  else if (kMaxAfter == 2 && after == 1) wait_vm_then_barrier<kLoads>();
  else wait_vm_then_barrier<0>();
}

// acc *= s for one 32x32 accumulator tile that lives in AGPRs: each element is
// read, scaled and written back in place through one temporary VGPR, so the
// rare rescale never needs a second copy of the accumulators.
__device__ __forceinline__ void scale_acc(f32x16& acc, float sc) {
#define DCP_SCALE1(i) "v_accvgpr_read_b32 %[t], %[a" #i "]\n\tv_mul_f32 %[t], %[t], %[s]\n\tv_accvgpr_write_b32 %[a" #i "], %[t]\n\t"
  float t;
  // leading pad: the accumulators may have just been written by an MFMA
  asm volatile("s_nop 15\n\t" DCP_SCALE1(0) DCP_SCALE1(1) DCP_SCALE1(2) DCP_SCALE1(3) DCP_SCALE1(4) DCP_SCALE1(5)
                   DCP_SCALE1(6) DCP_SCALE1(7) DCP_SCALE1(8) DCP_SCALE1(9) DCP_SCALE1(10) DCP_SCALE1(11)
                       DCP_SCALE1(12) DCP_SCALE1(13) DCP_SCALE1(14) DCP_SCALE1(15)
               : [t] "=&v"(t), [a0] "+a"(acc[0]), [a1] "+a"(acc[1]), [a2] "+a"(acc[2]),
                 [a3] "+a"(acc[3]), [a4] "+a"(acc[4]), [a5] "+a"(acc[5]), [a6] "+a"(acc[6]),
                 [a7] "+a"(acc[7]), [a8] "+a"(acc[8]), [a9] "+a"(acc[9]), [a10] "+a"(acc[10]),
                 [a11] "+a"(acc[11]), [a12] "+a"(acc[12]), [a13] "+a"(acc[13]), [a14] "+a"(acc[14]),
                 [a15] "+a"(acc[15])
               : [s] "v"(sc));
  asm volatile("s_nop 7" ::: "memory");   // before an MFMA reads the rewritten accumulators
#undef DCP_SCALE1
}

// Scalar (SMEM) read of a uniform 32-bit value: keeps page-table lookups off
// the vector-memory counter that tracks the in-flight tile loads.
__device__ __forceinline__ int32_t scalar_load(const int32_t* ptr) {
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

__device__ __forceinline__ float other_half(float v) {
  // value of lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// 16-byte direct-to-LDS load from a uniform base plus a per-lane 32-bit offset
// (the scalar-base form: no 64-bit per-lane address arithmetic).
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t off, uint32_t lds_addr) {
  // the base is wave-uniform by construction; say so, so that it always lands
  // in an SGPR pair (free when the compiler already knows)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(bu), "{m0}"(lds_addr) : "memory");
}

// Upper bound on KV chunks per request (each adds one partial to the workspace).
constexpr int kMaxSplits = 256;

template <int W, bool kAligned>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W), amdgpu_waves_per_eu(1, 1)))
stripe_attn_kernel(Params p) {
  using S = Shape<W>;
  __shared__ __align__(16) char smem[S::kLdsBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;          // which 8-element k half of an MFMA operand
  const int n = lane & 31;             // query row (MFMA column) owned by this lane

  // ---- work item: XCD-aware block order (the dispatcher sends block i to XCD
  // i % 8, so consecutive logical items share an XCD and its L2)
  int id = blockIdx.x;
  const int G = gridDim.x;
  if ((G & 7) == 0) id = (id & 7) * (G >> 3) + (id >> 3);
  const int mg = id % p.mgroups;
  const int rest = id / p.mgroups;
  const int split = rest % p.splits;
  const int b = rest / p.splits;

  const int32_t S_b = p.seq_len[b];
  const int32_t max_vis = count_rows(S_b, p.N, p.I, p.rank);   // rows the last query sees
  const int32_t row_lo = split * p.split_rows;
  int32_t row_hi = row_lo + p.split_rows;
  row_hi = row_hi < max_vis ? row_hi : max_vis;
  const int ntiles = row_hi > row_lo ? (row_hi - row_lo + kTile - 1) / kTile : 0;

  // ---- this lane's query row and its visible limit inside the split
  const int R = mg * 32 * W + wave * 32 + n;
  const bool valid = R < p.M;
  const int t = valid ? R / p.H : 0;
  int32_t lim = count_rows(S_b - p.q_len + t + 1, p.N, p.I, p.rank);
  if (!valid) lim = row_hi;
  lim = lim < row_hi ? lim : row_hi;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds row n, dims
  // 16*ks + 8*half .. +7 for every k-step
  bf16x8 qf[kKSteps];
  {
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(p.q + ((int64_t)b * p.M + (valid ? R : 0)) * kD);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = valid ? qrow[2 * ks + half] : bf16x8{};
  }

  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const char* zero = reinterpret_cast<const char*>(g_zero_row);
  const int32_t* bt_row = p.bt + (int64_t)b * p.bt_cols;

  // ---- page table of the split, one page id per lane, 64 pages at a time
  // (page-aligned tiles only: a tile lies inside one page)
  int32_t pt_base = kAligned ? row_lo / p.P : 0;
  int32_t vpt = -1;
  auto load_page_table = [&](int32_t base) {
    pt_base = base;
    const int32_t pi = base + lane;
    vpt = pi < p.bt_cols ? bt_row[pi] : -1;
    // Consume the loaded value right here, so the wait for this load happens
    // on this (rare) path; otherwise the compiler waits for every outstanding
    // vector-memory operation -- all in-flight tile loads -- at each later use.
    asm volatile("" : "+v"(vpt));
  };
  if (kAligned) load_page_table(pt_base);
  // base address of tile `it` (aligned path): its page, offset inside the page
  auto tile_base_of = [&](int it) -> const char* {
    const int32_t J = row_lo + it * kTile;
    const int32_t pi = J / p.P;
    if (pi - pt_base >= 64) load_page_table(pi);    // rare: long splits cross 64 pages
    const int32_t pg = __builtin_amdgcn_readlane(vpt, pi - pt_base);
    if (pg < 0 || pg >= p.num_pages) {
      if (lane == 0) flag_range(p.status);
      return nullptr;
    }
    return p.pool + ((int64_t)pg * p.P + (J % p.P)) * kRowBytes;
  };

  // A tile is "fast" when it is page-aligned and all 32 rows lie in the split:
  // its 32 rows are 36,864 contiguous bytes, so slot s of the padded LDS tile
  // (row s / 73, chunk s % 73) takes global chunk s - s / 73 of the tile; pad
  // chunks and slots past the tile fetch a neighbouring chunk of the same tile,
  // which is never read from LDS.
  auto tile_is_fast = [&](int it) -> bool {
    return kAligned && it < ntiles && row_hi - (row_lo + it * kTile) >= kTile;
  };
  auto fast_offset = [&](int k) -> uint32_t {
    const uint32_t s = (uint32_t)((k * W + wave) * 64 + lane);
    uint32_t g = s - ((s * 57457u) >> 22);          // s - floor(s / 73), exact for s < 4096
    g = g < (uint32_t)(kTile * kChunks - 1) ? g : (uint32_t)(kTile * kChunks - 1);
    return g * 16u;
  };
  // General loads (live tiles only): partial tiles and pages smaller than a
  // tile.  A slot that holds no token of the split (rows past the split end,
  // the pad chunk, slots past the tile) loads a chunk of the tile's first
  // row instead: finite data that the softmax masks to weight zero (or that
  // is never read), so no stale, unowned or NaN row reaches the MFMAs.
  auto load_tile_general = [&](int it) {
    const int stage = it % S::kStages;
    const int32_t J = row_lo + it * kTile;
    const int32_t rows_left = row_hi - J;          // >= 1 for a live tile
    const char* tb = nullptr;
    if (kAligned) tb = tile_base_of(it);
    const uint32_t lds_stage = lds0 + stage * S::kStageBytes;
#pragma unroll 1
    for (int k = 0; k < S::kLoads; ++k) {
      const int s = (k * W + wave) * 64 + lane;
      int tt = s / kRowSlots;
      int c = s - tt * kRowSlots;
      if (!(s < kTileSlots && tt < rows_left)) tt = 0;
      c = c < kChunks ? c : kChunks - 1;
      const char* src = zero;
      if (kAligned) {
        if (tb) src = tb + tt * kRowBytes + c * 16;
      } else {
        const int32_t j = J + tt;
        const int32_t pi = j / p.P;
        const int32_t pg = pi < p.bt_cols ? bt_row[pi] : -1;
        if (pg >= 0 && pg < p.num_pages) src = p.pool + ((int64_t)pg * p.P + j % p.P) * kRowBytes + c * 16;
        else flag_range(p.status);
      }
      dma16(src, lds_stage + (uint32_t)__builtin_amdgcn_readfirstlane((k * W + wave) * 1024));
    }
  };

  // ---- accumulators
  f32x16 oacc[kColBlocks];
#pragma unroll
  for (int cb = 0; cb < kColBlocks; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY;   // reference max (base-2 units) of this row
  float l_run = 0.f;         // this lane-half's share of the softmax denominator

  // per-lane LDS byte offsets inside a stage
  const int kq_off = (tau(n) * kRowSlots + half) * 16;          // + 32*ks
  const int g = lane >> 4, jl = lane & 15;
  const int v_off = ((4 * (jl >> 2) + (g >> 1)) * kRowSlots + 2 * (g & 1) + ((jl & 3) >> 1)) * 16 + (jl & 1) * 8;
  // tile-relative token of each of this lane's S^T registers (for masking)
  auto tok_of = [&](int i) { return 16 * (i >> 3) + 4 * (i & 3) + 2 * ((i >> 2) & 1) + half; };

  // ---- prologue: tiles 0 .. S-2 in flight, S^T of tile 0
#pragma unroll 1
  for (int it = 0; it < S::kStages - 1 && it < ntiles; ++it) {
    if (tile_is_fast(it)) {
      const char* tb = tile_base_of(it);
      const uint32_t lds_stage = lds0 + (it % S::kStages) * S::kStageBytes;
      if (tb) {
#pragma unroll 1
        for (int k = 0; k < S::kLoads; ++k)
          dma16_sbase(tb, fast_offset(k), lds_stage + (uint32_t)__builtin_amdgcn_readfirstlane((k * W + wave) * 1024));
      } else {
        load_tile_general(it);
      }
    } else {
      load_tile_general(it);
    }
  }
  const float c2 = p.c2;

#pragma unroll 1
  for (int it = 0; it < ntiles; ++it) {
    // Tile it is in LDS and every wave is done with tile it-1, whose stage
    // now receives tile it+S-1.
    const int after = ntiles - 1 - it;                 // live tiles after this one
    wait_tiles_then_barrier<S::kStages - 2, S::kLoads>(after);
    const int nt = it + S::kStages - 1;
    const bool fast = tile_is_fast(nt);
    const char* ntb = fast ? tile_base_of(nt) : nullptr;
    if (nt < ntiles && (!fast || ntb == nullptr)) load_tile_general(nt);
    const bool dma_in_pv = fast && ntb != nullptr;
    const uint32_t nlds = lds0 + (nt % S::kStages) * S::kStageBytes;
    const char* st = smem + (it % S::kStages) * S::kStageBytes;
    const int32_t J = row_lo + it * kTile;

    // -- S^T = K Q^T over the 576 latent dims (K fragments read kQkAhead steps ahead)
    f32x16 sacc = f32x16{};
    {
      const char* kb = st + kq_off;
      bf16x8 kf[kKSteps];
#pragma unroll
      for (int ks = 0; ks < kQkAhead; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(kb + 32 * ks);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks + kQkAhead < kKSteps) kf[ks + kQkAhead] = *reinterpret_cast<const bf16x8*>(kb + 32 * (ks + kQkAhead));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], sacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // -- online softmax in base 2.  Scores are masked only on tiles that
    // cross a row's visible limit; the row max is taken on the raw scores
    // (the scale is positive) and each weight costs one FMA and one exp2.
    const int32_t vis = lim - J;                       // visible rows of this tile
    if (__builtin_amdgcn_ballot_w64(vis < kTile) != 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = tok_of(i) < vis ? sacc[i] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
#pragma unroll
    for (int i = 3; i < 16; i += 2) mx = fmaxf(fmaxf(mx, sacc[i]), i + 1 < 16 ? sacc[i + 1] : -INFINITY);
    mx = fmaxf(mx, other_half(mx)) * c2;               // tile max in base-2 units
    const float m_new = fmaxf(m_run, mx);
    const bool move = m_new > m_run + 8.0f;             // move the reference only on a large jump
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) scale_acc(oacc[cb], alpha);
      l_run *= alpha;
      if (move) m_run = m_new;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
    bf16x8 pk[2];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c2, neg_m));
      psum += e;
      pk[i >> 3][i & 7] = (__bf16)e;
    }
    l_run += psum;

    // -- O^T += V^T P^T (V^T fragments by transpose reads, kPvAhead steps ahead),
    // with the loads of tile it+S-1 slotted under the MFMAs
    {
      const char* vb = st + v_off;
      auto vfrag = [&](int step) {
        const int cb = step >> 1, kk = step & 1;
        const char* a = vb + kk * (16 * kRowSlots * 16) + cb * 64;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 2 * kRowSlots * 16));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vf[2 * kColBlocks];
#pragma unroll
      for (int step = 0; step < kPvAhead; ++step) vf[step] = vfrag(step);
#pragma unroll
      for (int step = 0; step < 2 * kColBlocks; ++step) {
        if (step + kPvAhead < 2 * kColBlocks) vf[step + kPvAhead] = vfrag(step + kPvAhead);
        oacc[step >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[step], pk[step & 1], oacc[step >> 1], 0, 0, 0);
        if (step < S::kLoads && dma_in_pv)
          dma16_sbase(ntb, fast_offset(step), nlds + (uint32_t)__builtin_amdgcn_readfirstlane((step * W + wave) * 1024));
        __builtin_amdgcn_sched_barrier(0);
      }
      // the rest of the tile's loads when a wave issues more loads than PV steps
#pragma unroll 1
      for (int k = 2 * kColBlocks; k < S::kLoads; ++k)
        if (dma_in_pv)
          dma16_sbase(ntb, fast_offset(k), nlds + (uint32_t)__builtin_amdgcn_readfirstlane((k * W + wave) * 1024));
    }
  }
  // every load has landed by now; make that explicit before the LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: normalise and store this row's (o, lse)
  const float l_tot = l_run + other_half(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __builtin_amdgcn_logf(l_tot) : -INFINITY;
  float* orow;
  if (p.splits == 1) orow = p.o + ((int64_t)b * p.M + R) * kDV;
  else orow = p.ws_o + (((int64_t)split * p.B + b) * p.M + R) * kDV;
  if (valid) {
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 v;
        v.x = oacc[cb][4 * g4 + 0] * inv;
        v.y = oacc[cb][4 * g4 + 1] * inv;
        v.z = oacc[cb][4 * g4 + 2] * inv;
        v.w = oacc[cb][4 * g4 + 3] * inv;
        *reinterpret_cast<float4*>(orow + cb * 32 + 8 * g4 + 4 * half) = v;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (half == 0) {
      if (p.splits == 1) p.lse[(int64_t)b * p.M + R] = p.out_base2 ? lse2 : lse2 * kLn2;
      else p.ws_lse[((int64_t)split * p.B + b) * p.M + R] = lse2;
    }
  }
}

struct Plan {
  int W, mgroups, splits, split_rows;
  size_t ws_bytes;
};

int make_plan(const dcp_attn_args* a, Plan* pl) {
  if (a == nullptr || pl == nullptr) return DCP_EINVAL;
  if (!layout_ok(a->layout)) return DCP_EINVAL;
  if (a->rank < 0 || a->rank >= a->layout.n_stripes) return DCP_EINVAL;
  if (a->batch < 1 || a->q_len < 1 || a->n_heads < 1) return DCP_EINVAL;
  if (a->head_dim != kD || a->v_dim != kDV) return DCP_EUNSUPPORTED;
  if (a->bt_cols < 1 || a->num_pages < 1) return DCP_EINVAL;
  if (a->lse_base != 0 && a->lse_base != 1) return DCP_EINVAL;
  if (a->num_splits < 0) return DCP_EINVAL;
  const int64_t M = (int64_t)a->q_len * a->n_heads;
  const int64_t max_rows = (int64_t)a->bt_cols * a->layout.page_size;
  if (M > (1 << 20) || max_rows > 0x7fffffff - 64) return DCP_EUNSUPPORTED;
  if ((int64_t)a->layout.n_stripes * a->layout.interleave > 0x7fffffff) return DCP_EUNSUPPORTED;
  pl->W = M <= 32 ? 1 : (M <= 64 ? 2 : (M <= 96 ? 3 : 4));
  pl->mgroups = (int)ceil_div(M, 32 * pl->W);
  const int64_t tiles_max = ceil_div(max_rows, kTile);
  int64_t splits = a->num_splits;
  if (splits == 0) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
      int v = 0;
      if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    const int64_t base = (int64_t)a->batch * pl->mgroups;
    splits = ceil_div(cus, base);
  }
  if (splits > tiles_max) splits = tiles_max;
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits < 1) splits = 1;
  const int64_t tiles_per_split = ceil_div(tiles_max, splits);
  splits = ceil_div(tiles_max, tiles_per_split);
  pl->split_rows = (int)(tiles_per_split * kTile);
  pl->splits = (int)splits;
  if ((int64_t)a->batch * pl->splits * pl->mgroups > 0x7fffffff) return DCP_EUNSUPPORTED;
  // partials (o, lse) of every split
  pl->ws_bytes = pl->splits > 1 ? (size_t)pl->splits * a->batch * M * (kDV + 1) * sizeof(float) : 0;
  return DCP_OK;
}

template <int W>
int launch(const Params& prm, int64_t blocks, hipStream_t stream) {
  if (prm.P % kTile == 0)
    hipLaunchKernelGGL((stripe_attn_kernel<W, true>), dim3((unsigned)blocks), dim3(64 * W), 0, stream, prm);
  else
    hipLaunchKernelGGL((stripe_attn_kernel<W, false>), dim3((unsigned)blocks), dim3(64 * W), 0, stream, prm);
  return launch_status();
}

}  // namespace attn
}  // namespace dcp

using namespace dcp;
using namespace dcp::attn;

extern "C" int dcp_stripe_attn_workspace(const dcp_attn_args* args, size_t* bytes) {
  if (bytes == nullptr) return DCP_EINVAL;
  Plan pl;
  const int rc = make_plan(args, &pl);
  if (rc != DCP_OK) return rc;
  *bytes = pl.ws_bytes;
  return DCP_OK;
}

extern "C" int dcp_stripe_attn(const dcp_attn_args* a, void* stream) {
  Plan pl;
  const int rc = make_plan(a, &pl);
  if (rc != DCP_OK) return rc;
  if (a->q == nullptr || a->pool == nullptr || a->block_table == nullptr || a->seq_len == nullptr ||
      a->o == nullptr || a->lse == nullptr)
    return DCP_EINVAL;
  if (pl.ws_bytes > 0 && (a->workspace == nullptr || a->workspace_bytes < pl.ws_bytes)) return DCP_EINVAL;
  const int64_t M = (int64_t)a->q_len * a->n_heads;
  Params prm;
  prm.N = a->layout.n_stripes;
  prm.I = a->layout.interleave;
  prm.P = a->layout.page_size;
  prm.rank = a->rank;
  prm.B = a->batch;
  prm.q_len = a->q_len;
  prm.H = a->n_heads;
  prm.M = (int32_t)M;
  prm.W = pl.W;
  prm.mgroups = pl.mgroups;
  prm.splits = pl.splits;
  prm.split_rows = pl.split_rows;
  prm.q = (const __bf16*)a->q;
  prm.pool = (const char*)a->pool;
  prm.num_pages = a->num_pages;
  prm.bt = a->block_table;
  prm.bt_cols = a->bt_cols;
  prm.seq_len = a->seq_len;
  prm.c2 = a->scale * kLog2e;
  prm.out_base2 = a->lse_base;
  prm.o = a->o;
  prm.lse = a->lse;
  prm.ws_o = pl.splits > 1 ? (float*)a->workspace : nullptr;
  prm.ws_lse = pl.splits > 1 ? prm.ws_o + (size_t)pl.splits * a->batch * M * kDV : nullptr;
  prm.status = a->status;
  const int64_t blocks = (int64_t)a->batch * pl.splits * pl.mgroups;
  hipStream_t s = (hipStream_t)stream;
  int r;
  switch (pl.W) {
    case 1: r = launch<1>(prm, blocks, s); break;
    case 2: r = launch<2>(prm, blocks, s); break;
    case 3: r = launch<3>(prm, blocks, s); break;
    default: r = launch<4>(prm, blocks, s); break;
  }
  if (r != DCP_OK || pl.splits == 1) return r;
  // the chunks of each stripe row merge exactly like stripes (partial lse in base 2)
  return launch_lse_merge(pl.splits, (int64_t)a->batch * M, kDV, prm.ws_o, prm.ws_lse, 1, a->lse_base, a->o, a->lse, s);
}
