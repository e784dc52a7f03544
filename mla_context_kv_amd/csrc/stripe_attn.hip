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
//  * One workgroup of 8 wavefronts (two per SIMD) per (chunk of a request's
//    rows, group of up to 96 query rows = RB blocks of 32).  Heads are the N
//    side of the MFMA tiles, so one latent tile in LDS serves all of them.
//    Waves 0..RB-1 compute scores and softmax of one row block each, wave 3
//    issues the tile loads, waves 4..7 accumulate PV for 128 value columns.
//  * KV tiles of 32 tokens are streamed HBM -> LDS with 16-byte direct-to-LDS
//    loads into a 4-stage ring (two tiles in flight while one is scored and
//    the previous one accumulated); a tile's token rows are padded to 73
//    16-byte chunks so that the LDS access patterns below are bank-conflict
//    free.  The same LDS tile is the key (QK^T) and the value (PV): every KV
//    byte is read from HBM once.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (M = 32 tokens, N = 32 query
//    rows, K = 576 in 36 steps): score wave w owns query-row block w, whose Q
//    stays in its registers for the whole kernel.
//  * Online softmax in base 2 (scale * log2(e) folded in) by the same wave;
//    the reference max only moves when it grows by more than 2^8, so the O
//    rescale is rare and still exact, and a tile whose weights all stay below
//    2^8 never computes its max.  P (bf16) goes to a small LDS buffer.
//  * O^T += V^T P^T with the same MFMA (M = 32 value columns, N = 32 query
//    rows, K = 16 tokens), split by value columns, so each V^T fragment
//    (transpose read of the token-major tile) feeds RB MFMAs and the tile's
//    values are read from LDS once per workgroup, not once per row block.
//  * Work list: every request's rows are cut into chunks of whole tiles,
//    balanced over the batch so that the grid is one round of workgroups
//    (ragged lengths included); dcp_stripe_attn_multi lists the requests of
//    several ranks in one launch.  A request's only chunk writes (o_r, lse_r)
//    itself; otherwise each chunk writes an (o, lse) partial and a second
//    launch merges a request's chunks with the same exact LSE merge as across
//    stripes (the chunks are a disjoint partition of the stripe's rows).
//  * Variants that keep the merge exact (page "DCP", conditions for merging):
//    a sliding window only moves each row's first visible local row (and the
//    request's first tile); a logit softcap and a linear position bias
//    transform each score right after QK^T (their own kernel instantiation;
//    the bias uses the row's GLOBAL position); an attention sink adds one
//    zero-valued logit per head to the denominator of the request's first
//    chunk -- the caller gives it to one rank only.
#include <mutex>

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
constexpr int kRowBytes = kD * 2;       // 1152
constexpr int kWaves = 4;               // PV waves, one per SIMD
constexpr int kNW = 8;                  // wavefronts per workgroup
constexpr int kChunkGroup = 4;          // consecutive chunks kept on one XCD
constexpr int kLoaderWaveId = 3;
constexpr int kWaveCols = kDV / kWaves / 32;   // 4 value-column blocks of 32 per wave
constexpr int kMaxRB = 3;               // query-row blocks of 32 per workgroup

// Tile loads: instruction g fills the 64 tile slots from min(64 g, 2272), so
// the loader wave's 37 instructions cover a tile and a stage is exactly one
// tile (the last one overlaps the one before it and writes the same bytes
// again).
constexpr int kTileInsts = (kTileSlots + 63) / 64;   // 37
constexpr int kLastBase = kTileSlots - 64;
constexpr int kStageBytes = kTileSlots * 16;    // 37,376
// requests whose shapes a workgroup keeps in LDS (in the last tile stage, at
// the start of the kernel)
constexpr int kTableMax = 2304;
constexpr int kStages = 4;
// P^T rows: 4 chunks of 16 bytes, chunk kk*2 + lane half holding k-step kk;
// chunk c of row r sits at position c ^ ((r >> 2) & 3), so the 16-byte
// accesses of 16 consecutive rows hit disjoint banks.  P^T, the rescale
// factors and flags are double-buffered by tile parity (one barrier per
// tile).
constexpr int kPRow = 64;
constexpr int kPBuf = 3 * 32 * kPRow;                   // one buffer of 96 rows
constexpr int kPOff = kStages * kStageBytes;
constexpr int kAlphaOff = kPOff + 2 * kPBuf;            // [2][128] per-row rescale factor of a tile
constexpr int kInvOff = kAlphaOff + 2 * kMaxRB * 32 * 4;   // per-row 1 / l at the end
constexpr int kFlagOff = kInvOff + kMaxRB * 32 * 4;     // [2][16] one byte per row block: rescale
constexpr int kLdsBytes = kFlagOff + 32;
static_assert(kMaxRB * 32 * kPRow <= kPBuf, "one P^T buffer holds every row");
static_assert(kLdsBytes <= 163840, "LDS budget");
// epilogue staging: per PV wave one block of 32 rows x 128 columns (fp32),
// rows padded by 16 bytes, inside the tile ring
constexpr int kEpiPitch = kDV / kWaves + 4;            // floats per staged row
constexpr int kEpiWaveBytes = 32 * kEpiPitch * 4;      // 16,896
static_assert(kWaves * kEpiWaveBytes <= kStages * kStageBytes, "epilogue staging fits in the ring");
static_assert(kTileInsts <= 63, "vmcnt range");

// LDS operand prefetch depth (MFMA steps) of the QK^T and PV chains
#ifndef DCP_QK_AHEAD
#define DCP_QK_AHEAD 3
#endif
#ifndef DCP_PV_AHEAD
#define DCP_PV_AHEAD 4
#endif
constexpr int kQkAhead = DCP_QK_AHEAD;
constexpr int kPvAhead = DCP_PV_AHEAD;
static_assert(kQkAhead >= 1 && kQkAhead <= 15 && kPvAhead >= 1 && kPvAhead <= 7, "LDS counter range");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// A zero latent row (plus pad chunk): what a tile slot holds when its page id
// is out of range (the call also flags DCP_ERANGE), so a bad table never
// makes the kernel read outside the pool.
__device__ __align__(16) uint4 g_zero_row[kRowSlots];

// What differs between the ranks of one launch (one rank per dcp_stripe_attn
// call; up to kMaxRanks in dcp_stripe_attn_multi).
struct RankPtrs {
  const char* pool;
  const int32_t* bt;
  float* o;                         // final outputs (requests cut into one chunk)
  float* lse;
  uint2* rec;                       // packed records in place of o and lse, nullable
  const float* sinks;               // [H] natural-log sink logits, nullable
  const int32_t* sp_rows;           // sparse selection: local rows [B][sp_stride]
  const uint32_t* sp_bits;          //   which query tokens selected each entry (bit t)
  const int32_t* sp_count;          //   entries per request [B]
  int64_t num_pages;
  int32_t rank, bt_cols, sp_stride, pad;
};
constexpr int kMaxRanks = 16;
constexpr int kGroupChunkTiles = 512;   // longest chunk when a request's rows are cut into groups

struct Params {
  int32_t N, I, P;
  int32_t nr;                       // ranks in the launch: request v is request v % B of rank slot v / B
  int32_t B, q_len, H, M;          // M = q_len * H query rows per request
  int32_t RB, mgroups;
  int32_t slots;                    // chunk slots of the workspace (grid = slots * mgroups)
  int32_t forced_splits;            // > 0: that many chunks per request; 0: balanced chunks
  int32_t partials;                 // > 0: exactly this many chunks per request, each written
                                    // unmerged to o / lse as part (chunk, request) -- no combine
  int32_t target_chunks;            // balanced: at most this many chunks (when >= B)
  const __bf16* q;
  const int32_t* seq_len;
  float c2;                         // scale * log2(e)
  int32_t window;                   // > 0: a query at t sees t - window < p <= t
  float cap_in, cap_out;            // softcap: s -> cap_out * tanh(s * cap_in) (raw-score units)
  const float* slopes;              // [H] position-bias slopes (natural-log units), nullable
  int32_t sparse;                   // every rank has a sparse selection
  float inv_scale;                  // 1 / scale: a natural-log logit term in raw-score units
  int32_t out_base2;
  int32_t records;                  // outputs as packed records (bf16 o + float32 lse) in rk.rec
  int32_t o_bf16;                   // o (and unmerged parts) written as bf16, lse float32
  uint16_t* ws_o;                   // chunk partials: o as bf16 [slots][M][512], lse2 fp32 [slots][M]
  float* ws_lse;
  int32_t* table;                   // chunks per request [nr*B], first chunk of each request [nr*B]
  int32_t* status;
  RankPtrs rk[kMaxRanks];
};

// the DCP rank and sparse count of rank slot ri (a per-lane slot: selected
// from the wave-uniform parameters, so no parameter is indexed per lane)
__device__ __forceinline__ int32_t rank_id(const Params& p, int32_t ri) {
  int32_t r = p.rk[0].rank;
#pragma unroll
  for (int i = 1; i < kMaxRanks; ++i)
    if (i < p.nr && ri == i) r = p.rk[i].rank;
  return r;
}
__device__ __forceinline__ const int32_t* sp_count_of(const Params& p, int32_t ri) {
  const int32_t* c = p.rk[0].sp_count;
#pragma unroll
  for (int i = 1; i < kMaxRanks; ++i)
    if (i < p.nr && ri == i) c = p.rk[i].sp_count;
  return c;
}

// Record of query row R (= t * H + h) of request b, part kk, in 8-byte units
// (times kDV / 4 + 1): head-owner order [N][parts][B][q_len][H / N], so the
// block for owner d is one contiguous piece of the all-to-all send buffer.
__device__ __forceinline__ int64_t rec_index(const Params& p, int32_t kk, int32_t b, int32_t R) {
  const int32_t t = R / p.H, h = R - t * p.H;
  const int32_t Hl = p.H / p.N;
  const int32_t d = h / Hl, j = h - d * Hl;
  const int32_t K = p.partials > 0 ? p.partials : 1;
  return ((((int64_t)d * K + kk) * p.B + b) * p.q_len + t) * Hl + j;
}

// 32-bit layout arithmetic (positions < 2^31: seq_len is int32)
__device__ __forceinline__ int32_t count_rows(int32_t x, int32_t N, int32_t I, int32_t r) {
  if (x <= 0) return 0;
  const int32_t round = N * I;
  int32_t rem = x % round - r * I;
  rem = rem < 0 ? 0 : (rem > I ? I : rem);
  return (x / round) * I + rem;
}

// Inclusive prefix sum over the wave's 64 lanes (every lane active): shifts
// of 1, 2, 4 and 8 lanes inside each row of 16, then each row's total carried
// into the rows above it by the row broadcasts of lanes 15 and 31.  Cross-lane
// data paths of the VALU (DPP), a few cycles each, where a shuffle through
// the LDS crossbar waits on a memory round trip per step.
__device__ __forceinline__ int32_t wave_scan_i(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2 and 3
  return v;
}
// the wave's total (every lane active), wave-uniform
__device__ __forceinline__ int32_t wave_sum_i(int32_t v) { return __builtin_amdgcn_readlane(wave_scan_i(v), 63); }
__device__ __forceinline__ int32_t cdiv(int32_t a, int32_t b) { return (a + b - 1) / b; }

// Work list of one launch.  Request b's local rows (what its last query
// sees, from the first row its first query's window reaches, aligned down to
// a tile; or its selected entries) make tiles_b tiles of 32; the request is
// cut into n_b >= 1 chunks of cs_b = ceil(tiles_b / n_b) tiles (an empty
// request gets one empty chunk, which writes its zero output).  Requests of
// all the ranks of a launch are listed rank by rank (request v = request
// v % B of rank slot v / B).  With forced_splits = s: n_b = number of chunks
// of ceil(tiles_b / s) tiles.  Otherwise the chunks are balanced over the
// whole batch, n_b = ceil(tiles_b / C):
//  * fewer requests than target_chunks: C is the smallest of a few candidate
//    lengths that keeps the total under target_chunks (the last candidate,
//    ceil(total / (target - B)), always does), so the grid is one round;
//  * otherwise C = ceil(total / target), the mean share of a compute unit
//    (capped for row groups), at most target + B chunks.
// Chunks are numbered request by request; chunk c is this workgroup's (every
// wave finds it with wave-wide scans; the workgroup of chunk 0 also writes
// the table the chunk combine reads).
struct WorkItem {
  int32_t b, k, n, cs, rows;        // request, chunk of it, its chunks, chunk length (tiles), rows
  int32_t ft;                       // the request's first tile
  int32_t S;                        // the request's global length
  bool live;
};

// first local row any query of a request with S cached tokens can see
__device__ __forceinline__ int32_t first_row(const Params& p, int32_t S, int32_t rank) {
  return p.window > 0 ? count_rows(S - p.q_len + 1 - p.window, p.N, p.I, rank) : 0;
}

// What the chunks of (virtual) request v cover, from one load of its global
// length S (and of its count with a sparse selection): its local rows on its
// rank (the selected entries with a sparse selection), the tile of the first
// row any query sees, and the tiles from there on.
struct ReqShape {
  int32_t S, rows, ft, tiles;
};
__device__ __forceinline__ ReqShape req_shape(const Params& p, int32_t v) {
  const int32_t ri = v / p.B, b = v - ri * p.B;
  ReqShape r;
  r.S = p.seq_len[b];
  r.rows = p.sparse ? sp_count_of(p, ri)[b] : count_rows(r.S, p.N, p.I, rank_id(p, ri));
  r.ft = p.sparse ? 0 : first_row(p, r.S, rank_id(p, ri)) / 32;
  r.tiles = r.rows > 0 ? cdiv(r.rows, 32) - r.ft : 0;
  return r;
}

// Unmerged parts: chunk c is part c % k of request c / k (k = partials); a
// request of t tiles has parts of ceil(t / k) tiles, the last ones empty when
// t < k (an empty part writes o = 0, lse = -inf: zero weight in the merge).
__device__ __forceinline__ WorkItem part_work(const Params& p, int32_t c) {
  WorkItem w{0, 0, 0, 0, 0, 0, 0, false};
  const int32_t k = p.partials;
  w.b = c / k;
  w.live = w.b < p.nr * p.B;
  if (!w.live) return w;
  w.k = c - w.b * k;
  w.n = k;
  const ReqShape rs = req_shape(p, w.b);
  w.rows = rs.rows;
  w.ft = rs.ft;
  w.S = rs.S;
  const int32_t t = rs.tiles;
  w.cs = t > 0 ? cdiv(t, k) : 0;
  return w;
}

// `tab` (nullable): every request's (tiles, rows, first tile, length) in
// LDS, filled by the whole workgroup; without it (batches past its capacity)
// each wave loads what it needs as it goes.
__device__ __forceinline__ WorkItem find_work(const Params& p, int32_t c, bool write_table, const int4* tab) {
  const int lane = threadIdx.x & 63;
  const int32_t Bv = p.nr * p.B;                  // requests of all ranks in the launch
  auto tiles_of = [&](int32_t b0) -> int32_t {     // b0 = 64 * block
    const int32_t b = b0 + lane;
    if (b >= Bv) return 0;
    return tab != nullptr ? tab[b].x : req_shape(p, b).tiles;
  };
  int32_t C = 1;
  if (p.forced_splits == 0) {
    int32_t total = 0;
    for (int32_t b0 = 0; b0 < Bv; b0 += 64) total += tiles_of(b0);
    total = wave_sum_i(total);
    auto chunks_for = [&](int32_t len) -> int32_t {
      int32_t nc = 0;
      for (int32_t b0 = 0; b0 < Bv; b0 += 64)
        nc += b0 + lane < Bv ? max(cdiv(tiles_of(b0), len), 1) : 0;
      return wave_sum_i(nc);
    };
    const int32_t target = p.target_chunks;
    if (target <= Bv) {
      // at least one chunk per request anyway: chunks of the mean per-CU share,
      // so a long request is split and the rounds of workgroups stay balanced.
      // The row groups of one chunk share its tiles through L2 only while they
      // run in step, so with several groups a chunk is kept short.
      C = max(cdiv(total, target), 1);
      if (p.mgroups > 1) C = min(C, kGroupChunkTiles);
    } else {
      // the shortest chunk length whose chunks fit one round of `target`
      // workgroups: the count falls as the length grows, and the mean share
      // of target - Bv units always fits (at most one extra chunk per
      // request), so a bisection between the two finds it
      int32_t lo = max(cdiv(total, target), 1);
      if (chunks_for(lo) > target) {
        int32_t hi = max(cdiv(total, target - Bv), 1);
        ++lo;
        while (lo < hi) {
          const int32_t mid = lo + (hi - lo) / 2;
          if (chunks_for(mid) <= target) hi = mid;
          else lo = mid + 1;
        }
      }
      C = lo;
    }
  }
  WorkItem w{0, 0, 0, 0, 0, 0, 0, false};
  int32_t carry = 0;
  for (int32_t b0 = 0; b0 < Bv; b0 += 64) {
    const int32_t b = b0 + lane;
    const int32_t t = tiles_of(b0);
    int32_t nb = 0;
    if (b < Bv) {
      if (p.forced_splits > 0) nb = t > 0 ? cdiv(t, cdiv(t, p.forced_splits)) : 1;
      else nb = max(cdiv(t, C), 1);
    }
    const int32_t x = wave_scan_i(nb);             // inclusive scan over the wave
    const int32_t incl = carry + x, excl = incl - nb;
    if (write_table && b < Bv) {
      // Device lengths beyond the page table's capacity can ask for more
      // chunks than the workspace has slots: such chunks have no workgroup,
      // so the request is flagged (its output is unspecified) and its table
      // entry is cut to the slots that exist -- the combine never reads past
      // the workspace.
      const int32_t fit = incl <= p.slots ? nb : max(p.slots - excl, 0);
      if (fit != nb) flag_range(p.status);
      p.table[b] = fit;
      p.table[Bv + b] = excl;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(b < Bv && excl <= c && c < incl);
    if (hit != 0 && !w.live) {
      const int l = __builtin_ctzll(hit);
      w.live = true;
      w.b = b0 + l;
      w.k = c - __builtin_amdgcn_readlane(excl, l);
      w.n = __builtin_amdgcn_readlane(nb, l);
      if (tab != nullptr) {
        const int4 e = tab[w.b];
        w.rows = e.y;
        w.ft = e.z;
        w.S = e.w;
      } else {
        const ReqShape r = req_shape(p, w.b);
        w.rows = r.rows;
        w.ft = r.ft;
        w.S = r.S;
      }
      const int32_t tl = __builtin_amdgcn_readlane(t, l);
      w.cs = tl > 0 ? cdiv(tl, w.n) : 0;
      if (!write_table) break;
    }
    carry = __builtin_amdgcn_readlane(incl, 63);
  }
  return w;
}

// The one-round plan of a launch with fewer requests than its round of
// workgroups and at most 256 of them (one rank's call on a decode batch of up
// to 256 requests), from registers: each lane holds the shapes of requests
// lane, lane + 64, ..., read from the request table once, and every step of
// the search (the total, the chunk counts of each candidate length, the scan,
// the request of chunk c and its shape) runs on them -- the same chunk length
// and numbering as find_work, with no further LDS round trips.
constexpr int kSmallPerLane = 4;
__device__ __forceinline__ WorkItem find_work_small(const Params& p, int32_t c, bool write_table, const int4* tab) {
  const int lane = threadIdx.x & 63;
  const int32_t Bv = p.nr * p.B;
  int4 e[kSmallPerLane];
  int32_t tsum = 0;
#pragma unroll
  for (int k = 0; k < kSmallPerLane; ++k) {
    const int32_t v = 64 * k + lane;
    e[k] = v < Bv ? tab[v] : make_int4(0, 0, 0, 0);
    tsum += e[k].x;
  }
  const int32_t total = wave_sum_i(tsum);
  const int32_t target = p.target_chunks;
  auto chunks_for = [&](int32_t len) -> int32_t {
    int32_t nc = 0;
#pragma unroll
    for (int k = 0; k < kSmallPerLane; ++k)
      nc += 64 * k + lane < Bv ? max(cdiv(e[k].x, len), 1) : 0;
    return wave_sum_i(nc);
  };
  // the shortest chunk length whose chunks fit the round (find_work's rule)
  int32_t C = max(cdiv(total, target), 1);
  if (chunks_for(C) > target) {
    int32_t hi = max(cdiv(total, target - Bv), 1);
    ++C;
    while (C < hi) {
      const int32_t mid = C + (hi - C) / 2;
      if (chunks_for(mid) <= target) hi = mid;
      else C = mid + 1;
    }
  }
  WorkItem w{0, 0, 0, 0, 0, 0, 0, false};
  int32_t carry = 0;
#pragma unroll
  for (int k = 0; k < kSmallPerLane; ++k) {
    if (64 * k >= Bv) break;
    const int32_t v = 64 * k + lane;
    const int32_t t = e[k].x;
    const int32_t nb = v < Bv ? max(cdiv(t, C), 1) : 0;
    const int32_t incl = carry + wave_scan_i(nb), excl = incl - nb;
    if (write_table && v < Bv) {
      // entries cut to the workspace's slots, as in find_work
      const int32_t fit = incl <= p.slots ? nb : max(p.slots - excl, 0);
      if (fit != nb) flag_range(p.status);
      p.table[v] = fit;
      p.table[Bv + v] = excl;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(v < Bv && excl <= c && c < incl);
    if (hit != 0 && !w.live) {
      const int l = __builtin_ctzll(hit);
      w.live = true;
      w.b = 64 * k + l;
      w.k = c - __builtin_amdgcn_readlane(excl, l);
      w.n = __builtin_amdgcn_readlane(nb, l);
      w.rows = __builtin_amdgcn_readlane(e[k].y, l);
      w.ft = __builtin_amdgcn_readlane(e[k].z, l);
      w.S = __builtin_amdgcn_readlane(e[k].w, l);
      const int32_t tl = __builtin_amdgcn_readlane(t, l);
      w.cs = tl > 0 ? cdiv(tl, w.n) : 0;
      if (!write_table) break;
    }
    carry = __builtin_amdgcn_readlane(incl, 63);
  }
  return w;
}

// Workspace slot of chunk c's partial (o, lse): the chunks of each group of
// kChunkGroup (one XCD's consecutive chunks) go to kChunkGroup regions of the
// workspace, slot (c mod kChunkGroup) * (slots / kChunkGroup) + c / kChunkGroup.
// A bijection on the slots (a multiple of kChunkGroup), so every chunk keeps a
// slot of its own; the attention kernel writes and the chunk combine reads
// through it.  The XCDs' partial writes then interleave in memory at the
// grain of one chunk instead of one group of chunks, which measured faster.
__device__ __forceinline__ int64_t part_slot(const Params& p, int64_t c) {
  return (c % kChunkGroup) * (p.slots / kChunkGroup) + c / kChunkGroup;
}

// Chunk classes of the many-request plan: chunks of about 2^(30 - key)
// tiles, key 31 for an empty request.  The plan numbers chunks class by
// class, longest first (and request by request inside a class), so the
// longest chunks take the first blocks of the launch and the short ones fill
// the compute units that free up later: a longest-first order for launches of
// several rounds of workgroups.
constexpr int kClasses = 32;
__device__ __forceinline__ int32_t chunk_class(int32_t cs) { return cs > 0 ? 30 - (31 - __builtin_clz(cs)) : 31; }

// The many-request plan (more requests than workgroups per round): chunks of
// the mean per-CU share C, numbered by class (longest chunks first) and in
// request order within a class.  `tab` holds every request's shape, `cls`
// [kClasses] the chunks of each class (filled by the workgroup).  Each wave
// finds chunk c itself, with one scan over the requests per 64 of them: the
// form for a few hundred requests.
__device__ __forceinline__ WorkItem find_work_classes(const Params& p, int32_t c, const int4* tab,
                                                      const int32_t* cls, int32_t C) {
  const int lane = threadIdx.x & 63;
  const int32_t Bv = p.nr * p.B;
  WorkItem w{0, 0, 0, 0, 0, 0, 0, false};
  // the class of chunk c, from the per-class counts
  const int32_t cnt = lane < kClasses ? cls[lane] : 0;
  const int32_t x = wave_scan_i(cnt);
  const uint64_t in_class = __builtin_amdgcn_ballot_w64(x - cnt <= c && c < x);
  if (in_class == 0) return w;                   // past the last chunk
  const int key = __builtin_ctzll(in_class);
  const int32_t r = c - (__builtin_amdgcn_readlane(x, key) - __builtin_amdgcn_readlane(cnt, key));
  // the request of the class's r-th chunk, in request order
  int32_t carry = 0;
  for (int32_t b0 = 0; b0 < Bv; b0 += 64) {
    const int32_t b = b0 + lane;
    const int32_t t = b < Bv ? tab[b].x : 0;
    const int32_t nb = max(cdiv(t, C), 1);
    const int32_t cs = t > 0 ? cdiv(t, nb) : 0;
    const int32_t mine = b < Bv && chunk_class(cs) == key ? nb : 0;
    const int32_t y = wave_scan_i(mine);
    const int32_t incl = carry + y, excl = incl - mine;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(mine > 0 && excl <= r && r < incl);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      w.live = true;
      w.b = b0 + l;
      w.k = r - __builtin_amdgcn_readlane(excl, l);
      w.n = __builtin_amdgcn_readlane(nb, l);
      w.cs = __builtin_amdgcn_readlane(cs, l);
      const int4 e = tab[w.b];
      w.rows = e.y;
      w.ft = e.z;
      w.S = e.w;
      return w;
    }
    carry = __builtin_amdgcn_readlane(incl, 63);
  }
  return w;
}

// The same numbering found by the whole workgroup, for many requests (above
// kBlockFind): each thread takes a contiguous run of requests, so one scan
// over the threads finds the request of chunk c, where a wave alone would
// scan 64 requests at a time.  Called by every thread of the workgroup (it
// holds two barriers); aux[1 + key] holds the chunks of each class,
// aux[kAuxWaves ..] and aux[kAuxFound ..] are scratch.
constexpr int kBlockFind = 512;
constexpr int kAuxWaves = 1 + kClasses;          // [kNW]: chunks of the class in each wave's runs
constexpr int kAuxFound = kAuxWaves + kNW;       // [4]: request, chunk of it, its chunks, chunk length
static_assert(kTableMax * 16 + (kAuxFound + 4) * 4 <= kStageBytes, "request table and its scratch fit one stage");
__device__ __forceinline__ WorkItem find_work_block(const Params& p, int32_t c, const int4* tab, int32_t* aux,
                                                    int32_t C) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t Bv = p.nr * p.B;
  // the class of chunk c and its rank r in the class, from the per-class counts
  const int32_t cnt = lane < kClasses ? aux[1 + lane] : 0;
  const int32_t x = wave_scan_i(cnt);
  const uint64_t in_class = __builtin_amdgcn_ballot_w64(x - cnt <= c && c < x);
  const int key = in_class != 0 ? __builtin_ctzll(in_class) : -1;      // -1: past the last chunk
  const int32_t r = key >= 0 ? c - (__builtin_amdgcn_readlane(x, key) - __builtin_amdgcn_readlane(cnt, key)) : 0;
  // the chunks of class `key` in this thread's run of requests
  const int32_t q = (Bv + 64 * kNW - 1) / (64 * kNW);
  const int32_t v0 = (int32_t)threadIdx.x * q;
  int32_t s = 0;
  for (int32_t j = 0; j < q; ++j) {
    const int32_t v = v0 + j;
    if (v < Bv) {
      const int32_t tv = tab[v].x;
      const int32_t nb = max(cdiv(tv, C), 1);
      if (chunk_class(tv > 0 ? cdiv(tv, nb) : 0) == key) s += nb;
    }
  }
  const int32_t incl = wave_scan_i(s);
  if (lane == 63) aux[kAuxWaves + wave] = incl;
  if (threadIdx.x == 0) aux[kAuxFound] = -1;
  __syncthreads();
  int32_t excl = incl - s;
  for (int w = 0; w < wave; ++w) excl += aux[kAuxWaves + w];
  if (s > 0 && excl <= r && r < excl + s) {
    // the one thread whose run holds chunk r of the class
    int32_t acc = excl;
    for (int32_t j = 0; j < q; ++j) {
      const int32_t v = v0 + j;
      if (v >= Bv) break;
      const int32_t tv = tab[v].x;
      const int32_t nb = max(cdiv(tv, C), 1);
      const int32_t cs = tv > 0 ? cdiv(tv, nb) : 0;
      if (chunk_class(cs) != key) continue;
      if (r < acc + nb) {
        aux[kAuxFound] = v;
        aux[kAuxFound + 1] = r - acc;
        aux[kAuxFound + 2] = nb;
        aux[kAuxFound + 3] = cs;
        break;
      }
      acc += nb;
    }
  }
  __syncthreads();
  WorkItem w{0, 0, 0, 0, 0, 0, 0, false};
  const int32_t vf = aux[kAuxFound];
  if (vf >= 0) {
    w.live = true;
    w.b = vf;
    w.k = aux[kAuxFound + 1];
    w.n = aux[kAuxFound + 2];
    w.cs = aux[kAuxFound + 3];
    const int4 e = tab[vf];
    w.rows = e.y;
    w.ft = e.z;
    w.S = e.w;
  }
  return w;
}

// MFMA row m of the QK^T A operand <-> token of the tile.  Within each group
// of 16, rows are transposed 4x4 so that a transpose read of V (4 tokens at
// once) touches 4 token rows 4 apart, which the 73-chunk row padding puts in
// disjoint LDS banks.
__device__ __forceinline__ int tau(int m) { return 16 * (m >> 4) + 4 * (m & 3) + ((m >> 2) & 3); }

__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(lds_addr) : "memory");
}

// 16-byte direct-to-LDS load from a uniform base plus a per-lane 32-bit offset
// (the scalar-base form: no 64-bit per-lane address arithmetic).  The KV
// stream is read once, so the load is marked non-temporal: it does not push
// the chunk partials and outputs out of L2 and the memory-side cache.
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t off, uint32_t lds_addr) {
  // the base is wave-uniform by construction; say so, so that it always lands
  // in an SGPR pair (free when the compiler already knows)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(bu), "{m0}"(lds_addr) : "memory");
}

// this wave's loads older than the N most recent ones and its LDS accesses
// are done, then barrier
template <int N>
__device__ __forceinline__ void wait_vm_then_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait until only the loads of the `after` most recent tiles (kPerTile per
// wave each) are in flight, then barrier.  Tiles past the chunk issue no
// loads, so near the end fewer tiles are in flight and the count drops with
// them.  A count above the counter's range waits for a few loads more.
template <int kPerTile>
__device__ __forceinline__ void wait_tiles_then_barrier(int after) {
  constexpr int kTwo = 2 * kPerTile < 63 ? 2 * kPerTile : 63;
  if (after >= 2) wait_vm_then_barrier<kTwo>();
  else if (after == 1) wait_vm_then_barrier<kPerTile>();
  else wait_vm_then_barrier<0>();
}

// this wave's LDS accesses are done
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// LDS writes of this wave done, then barrier
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float other_half(float v) {
  // value of lane l ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}


// Eight wavefronts, two per SIMD, with split roles: waves 0..RB-1 compute
// the scores and softmax of one block of 32 query rows each, wave 3 issues
// the tile loads, waves 4..7 accumulate PV for 128 value columns each -- so
// one wave's softmax and LDS waits overlap the other wave's MFMAs on the
// same SIMD; one barrier per tile, P^T double-buffered.
template <int RB, bool kAligned, bool kLogit>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * kNW, 64 * kNW), amdgpu_waves_per_eu(2, 2)))
stripe_attn_kernel(Params p) {
  static_assert(RB >= 1 && RB <= kMaxRB, "query-row blocks");
  __shared__ __align__(16) char smem[kLdsBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;          // which 8-element k half of an MFMA operand
  const int n = lane & 31;             // query row (MFMA column) owned by this lane
  const bool qk_wave = wave < RB;      // owns query-row block `wave` for QK^T and softmax
  const bool pv_wave = wave >= 4;
  const int cgrp = wave - 4;           // PV wave: value columns 128*cgrp .. +127

  // ---- work item: XCD-aware block order.  The dispatcher sends block i to
  // XCD i % 8.  Groups of kChunkGroup consecutive chunks go to the XCDs in
  // turn (chunk c to XCD (c / kChunkGroup) % 8): the live chunks (numbered
  // first; a plan may hold more slots than a call's lengths fill) spread over
  // every XCD, while a request's neighbouring chunks share an XCD and its L2
  // (its queries are read there once).  The row groups of one chunk are
  // consecutive blocks of that XCD, so they run side by side and share each
  // KV tile through its L2.  (The plan makes the slot count a multiple of
  // 8 * kChunkGroup, so the map is a bijection.)
  const int bid = blockIdx.x;
  const int bx = bid & 7, bk = bid >> 3;
  const int mg = bk % p.mgroups;
  const int bj = bk / p.mgroups;                 // this block's chunk is the bj-th on its XCD
  const int32_t chunk = ((bj / kChunkGroup) * 8 + bx) * kChunkGroup + bj % kChunkGroup;
  // Every request's shape, loaded once by the whole workgroup into the last
  // tile stage (the loader first fills it after the loop's first barrier, and
  // every wave is done with the table before that barrier).
  const int32_t Bv = p.nr * p.B;
  const int4* table = nullptr;
  // many requests per round of workgroups: chunks of the mean per-CU share,
  // numbered longest class first
  const bool classes = p.partials == 0 && p.forced_splits == 0 && p.target_chunks <= Bv && Bv <= kTableMax;
  int32_t C = 1;
  if (p.partials == 0 && Bv <= kTableMax) {
    int4* t = reinterpret_cast<int4*>(smem + (kStages - 1) * kStageBytes);
    int32_t* const aux = reinterpret_cast<int32_t*>(t + kTableMax);   // [0] total tiles, [1 + key] chunks
    if (classes) {
      if (threadIdx.x < 1 + kClasses) aux[threadIdx.x] = 0;
      __syncthreads();
    }
    int32_t mine = 0;
    for (int v = threadIdx.x; v < Bv; v += 64 * kNW) {
      const ReqShape r = req_shape(p, v);
      t[v] = make_int4(r.tiles, r.rows, r.ft, r.S);
      mine += r.tiles;
    }
    if (classes) {
      mine = wave_sum_i(mine);
      if (lane == 0) atomicAdd(&aux[0], mine);
    }
    __syncthreads();
    table = t;
    if (classes) {
      C = max(cdiv(aux[0], p.target_chunks), 1);
      if (p.mgroups > 1) C = min(C, kGroupChunkTiles);
      for (int v = threadIdx.x; v < Bv; v += 64 * kNW) {
        const int32_t tv = t[v].x;
        const int32_t nb = max(cdiv(tv, C), 1);
        atomicAdd(&aux[1 + chunk_class(tv > 0 ? cdiv(tv, nb) : 0)], nb);
      }
      __syncthreads();
    }
  }
  WorkItem wi;
  if (p.partials > 0) {
    wi = part_work(p, chunk);
  } else if (__builtin_expect(classes, 0)) {   // (placed out of the way of the common path's code)
    int32_t* const aux = reinterpret_cast<int32_t*>(smem + (kStages - 1) * kStageBytes) + 4 * kTableMax;
    wi = Bv > kBlockFind ? find_work_block(p, chunk, table, aux, C)      // (uniform in the workgroup)
                         : find_work_classes(p, chunk, table, aux + 1, C);
    if (p.table != nullptr && mg == 0 && wave == 0 && lane == 0) {
      // the chunk table the combine reads: each request's first chunk writes
      // its entry (cut to the slots there are; chunks without a workgroup
      // make the call flagged), and the workgroup of chunk 0 checks the count
      if (wi.live && wi.k == 0) {
        const int32_t fit = chunk + wi.n <= p.slots ? wi.n : p.slots - chunk;
        if (fit != wi.n) flag_range(p.status);
        p.table[wi.b] = fit;
        p.table[Bv + wi.b] = chunk;
      }
      if (chunk == 0) {
        int32_t tot = 0;
        for (int key = 0; key < kClasses; ++key) tot += aux[1 + key];
        if (tot > p.slots) flag_range(p.status);
      }
    }
  } else if (table != nullptr && p.forced_splits == 0 && p.target_chunks > Bv && Bv <= 64 * kSmallPerLane) {
    wi = find_work_small(p, chunk, p.table != nullptr && chunk == 0 && mg == 0 && wave == 0, table);
  } else {
    wi = find_work(p, chunk, p.table != nullptr && chunk == 0 && mg == 0 && wave == 0, table);
  }
  if (!wi.live) return;                // past the last chunk (the same in every wave)
  const int32_t ri = wi.b / p.B;       // rank slot of the launch
  const int b = wi.b - ri * p.B;       // request
  const RankPtrs& rk = p.rk[ri];
  // the request's only chunk, and every unmerged part, writes the output itself
  const bool direct = wi.n == 1 || p.partials > 0;
  const int64_t out_row0 = ((p.partials > 0 ? (int64_t)wi.k * p.B : 0) + b) * p.M;   // first output row

  const int32_t S_b = wi.S;
  const int32_t max_vis = wi.rows;     // rows the last query sees
  // sparse selection: the chunks run over entries of the request's list of
  // selected local rows; with several drafts each entry carries the drafts
  // that selected it
  const bool sparse = p.sparse != 0;
  const bool sparse_bits = sparse && p.q_len > 1;
  const int64_t sp_base = sparse ? (int64_t)b * rk.sp_stride : 0;
  const int32_t row_lo = (wi.ft + wi.k * wi.cs) * kTile;
  int32_t row_hi = row_lo + wi.cs * kTile;
  row_hi = row_hi < max_vis ? row_hi : max_vis;
  const int ntiles = row_hi > row_lo ? (row_hi - row_lo + kTile - 1) / kTile : 0;
  const int row0 = mg * 32 * RB;       // first query row of this workgroup

  // ---- QK wave: its query row and the row's visible limit inside the chunk
  const int R = row0 + wave * 32 + n;
  const bool valid = qk_wave && R < p.M;
  const int t = valid ? R / p.H : 0;
  int32_t lim = sparse ? row_hi : count_rows(S_b - p.q_len + t + 1, p.N, p.I, rk.rank);
  if (!valid) lim = row_hi;
  lim = lim < row_hi ? lim : row_hi;
  // first visible row (sliding window): rows below it are masked
  int32_t low = 0;
  if (valid && p.window > 0) low = count_rows(S_b - p.q_len + t + 1 - p.window, p.N, p.I, rk.rank);

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds row n, dims
  // 16*ks + 8*half .. +7 for every k-step (QK waves, loaded on their path)
  bf16x8 qf[kKSteps];
  auto load_q = [&]() {
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(p.q + ((int64_t)b * p.M + (valid ? R : 0)) * kD);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = valid ? qrow[2 * ks + half] : bf16x8{};
  };

  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  if (threadIdx.x < 8) reinterpret_cast<uint32_t*>(smem + kFlagOff)[threadIdx.x] = 0;   // ordered by the first barrier
  const char* zero = reinterpret_cast<const char*>(g_zero_row);
  const int32_t* bt_row = rk.bt + (int64_t)b * rk.bt_cols;

  // ---- page table of the chunk, one page id per lane, 64 pages at a time
  // (page-aligned tiles only: a tile lies inside one page)
  int32_t pt_base = kAligned ? row_lo / p.P : 0;
  int32_t vpt = -1;
  auto load_page_table = [&](int32_t base) {
    pt_base = base;
    const int32_t pi = base + lane;
    vpt = pi < rk.bt_cols ? bt_row[pi] : -1;
    // Consume the loaded value right here, so the wait for this load happens
    // on this (rare) path; otherwise the compiler waits for every outstanding
    // vector-memory operation -- all in-flight tile loads -- at each later use.
    asm volatile("" : "+v"(vpt));
  };
  // base address of tile `it` (aligned path): its page, offset inside the page
  auto tile_base_of = [&](int it) -> const char* {
    const int32_t J = row_lo + it * kTile;
    const int32_t pi = J / p.P;
    if (pi - pt_base >= 64) load_page_table(pi);    // rare: long chunks cross 64 pages
    const int32_t pg = __builtin_amdgcn_readlane(vpt, pi - pt_base);
    if (pg < 0 || pg >= rk.num_pages) {
      if (lane == 0) flag_range(p.status);
      return nullptr;
    }
    return rk.pool + ((int64_t)pg * p.P + (J % p.P)) * kRowBytes;
  };

  // the loader wave issues all 37 loads of a tile
  constexpr int kMyLoads = kTileInsts;
  const bool loads_here = wave == kLoaderWaveId;
  // first tile slot that load j fills
  auto load_slot0 = [&](int j) -> int {
    const int s0 = 64 * j;
    return s0 < kLastBase ? s0 : kLastBase;
  };
  // A tile is "fast" when it is page-aligned and all 32 rows lie in the chunk:
  // its 32 rows are 36,864 contiguous bytes, so slot s of the padded LDS tile
  // (row s / 73, chunk s % 73) takes global chunk s - s / 73 of the tile; the
  // pad chunks fetch a neighbouring chunk of the same tile, never read from LDS.
  auto tile_is_fast = [&](int it) -> bool {
    return kAligned && !sparse && it < ntiles && row_hi - (row_lo + it * kTile) >= kTile;
  };
  auto fast_offset = [&](int k) -> uint32_t {
    const uint32_t s = (uint32_t)(load_slot0(k) + lane);
    uint32_t g = s - ((s * 57457u) >> 22);          // s - floor(s / 73), exact for s < 4096
    g = g < (uint32_t)(kTile * kChunks - 1) ? g : (uint32_t)(kTile * kChunks - 1);
    return g * 16u;
  };
  // General loads (live tiles only): partial tiles, pages smaller than a
  // tile and sparse selections.  Lane l < 32 first finds the address of the
  // tile's row l (one round of dependent loads for the whole tile); each slot
  // then takes its row's address from that lane.  A slot that holds no token
  // of the chunk (rows past the chunk end) loads a 16-byte piece of the tile's first
  // row instead, and the pad chunk loads chunk 71 of its row: finite data
  // that the softmax masks to weight zero (or that is never read), so no
  // stale, unowned or NaN row reaches the MFMAs.  A row whose page is out of
  // range reads the zero row (and flags DCP_ERANGE).
  auto load_tile_general = [&](int it) {
    if (!loads_here) return;
    const int32_t J = row_lo + it * kTile;
    const int32_t rows_left = row_hi - J;          // >= 1 for a live tile
    const int l = lane & 31;
    const int tl = l < rows_left ? l : 0;
    const char* rowp = zero;
    if (kAligned && !sparse) {
      const char* tb = tile_base_of(it);
      if (tb) rowp = tb + tl * kRowBytes;
    } else {
      const int32_t j = sparse ? rk.sp_rows[sp_base + J + tl] : J + tl;
      const int32_t pi = j / p.P;
      const int32_t pg = j >= 0 && pi < rk.bt_cols ? bt_row[pi] : -1;
      if (pg >= 0 && pg < rk.num_pages) rowp = rk.pool + ((int64_t)pg * p.P + j % p.P) * kRowBytes;
      else flag_range(p.status);
    }
    const uint64_t ra = reinterpret_cast<uint64_t>(rowp);
    const uint32_t ra_lo = (uint32_t)ra, ra_hi = (uint32_t)(ra >> 32);
    const uint32_t lds_stage = lds0 + (it % kStages) * kStageBytes;
#pragma unroll 1
    for (int k = 0; k < kMyLoads; ++k) {
      const int s0 = load_slot0(k);
      const int s = s0 + lane;
      int tt = s / kRowSlots;
      int c = s - tt * kRowSlots;
      if (tt >= rows_left) tt = 0;
      c = c < kChunks ? c : kChunks - 1;
      const uint64_t a = ((uint64_t)(uint32_t)__shfl((int)ra_hi, tt, 64) << 32) | (uint32_t)__shfl((int)ra_lo, tt, 64);
      dma16(reinterpret_cast<const char*>(a) + c * 16, lds_stage + (uint32_t)__builtin_amdgcn_readfirstlane(s0 * 16));
    }
  };

  // ---- accumulators of a PV wave: its value columns of every row block
  f32x16 oacc[RB][kWaveCols];
  auto init_o = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < kWaveCols; ++cb) oacc[rb][cb] = f32x16{};
  };
  float m_run = -INFINITY;   // QK wave: reference max (base-2 units) of its row
  float l_run = 0.f;         // QK wave: this lane-half's share of the softmax denominator

  // per-lane LDS byte offsets
  const int kq_off = (tau(n) * kRowSlots + half) * 16;          // + 32*ks
  const int g4 = lane >> 4, jl = lane & 15;
  const int v_off = ((4 * (jl >> 2) + (g4 >> 1)) * kRowSlots + 2 * (g4 & 1) + ((jl & 3) >> 1)) * 16 + (jl & 1) * 8 +
                    cgrp * kWaveCols * 64;                        // + cb*64, + 16 token rows per k-step
  // P^T chunk kk*2 + half of row r (swizzled), in buffer `buf`
  auto p_addr = [&](int buf, int r, int kk) -> char* {
    return smem + kPOff + buf * kPBuf + r * kPRow + (((kk * 2 + half) ^ ((r >> 2) & 3)) * 16);
  };
  // tile-relative token of each of this lane's S^T registers (for masking)
  auto tok_of = [&](int i) { return 16 * (i >> 3) + 4 * (i & 3) + 2 * ((i >> 2) & 1) + half; };

  const float c2 = p.c2;
  // Logit transforms on the raw scores of the tile starting at local row j0
  // (kept in units where x * c2 is the logit in base 2), before any masking.
  // Softcap: tanh(y) = 1 - 2 / (e^2y + 1), one exp and one reciprocal; it
  // saturates to +-1 (e^2y = inf or 0), and its absolute error (a few ulp of
  // 1) is a negligible shift of the capped score.  Position bias: + slope *
  // (p - t) with p the row's global position p = floor(j / I) I N + r I + j mod I.
  float bias_raw = 0.f;                 // this row's slope in raw-score units
  int32_t q_pos = 0;                    // this row's query position
  if constexpr (kLogit) {
    if (p.slopes != nullptr && valid) bias_raw = p.slopes[R % p.H] * p.inv_scale;
    q_pos = S_b - p.q_len + t;
  }
  auto cap = [&](f32x16& x, int32_t j0) {
    if constexpr (kLogit) {
      if (p.cap_out > 0.f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e2y = __builtin_amdgcn_exp2f(x[i] * p.cap_in * (2.0f * kLog2e));
          x[i] = p.cap_out * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e2y + 1.0f));
        }
      }
      if (p.slopes != nullptr) {
        const int32_t round = p.N * p.I;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t j = j0 + tok_of(i);
          const int32_t pos = (j / p.I) * round + rk.rank * p.I + j % p.I;
          x[i] += bias_raw * (float)(pos - q_pos);
        }
      }
    }
  };

  // S^T = K Q^T of the tile in stage `st` over the 576 latent dims (K
  // fragments read kQkAhead steps ahead).  One accumulator: the matrix core
  // chains dependent MFMAs on their accumulator, and a second chain (tried)
  // only costs 16 registers and a 16-add reduction per tile.
  auto qk = [&](const char* st) -> f32x16 {
    f32x16 acc = f32x16{};
    const char* kb = st + kq_off;
    bf16x8 kf[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kQkAhead; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(kb + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + kQkAhead < kKSteps) kf[ks + kQkAhead] = *reinterpret_cast<const bf16x8*>(kb + 32 * (ks + kQkAhead));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
  };

  // Online softmax of one tile in base 2 (QK waves), in kParts pieces.
  // Scores are masked
  // only on tiles that cross a row's visible limit; the row max is taken on
  // the raw scores (the scale is positive); each weight costs one FMA and one
  // exp2.  The pieces publish the row block's rescale flag and factors (when
  // the reference max moves); P^T stays in registers until the next tile.
  constexpr int kParts = 11;
  f32x16 sacc;
  int32_t vis = 0, vlo = 0;             // tile-relative visible rows [vlo, vis)
  int32_t tj0 = 0;                      // the tile's first row (entry, with a sparse selection)
  float mx = 0.f, neg_m = 0.f, psum = 0.f;
  bf16x8 pk[2];
  int sbuf = 0;                       // buffer of the factors and flags the pieces publish
  auto softmax_part = [&](int part) {
    if (part == 0) {
      if (sparse_bits) {
        // several drafts: an entry is visible to the drafts that selected it
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int e = tok_of(i);
          const bool sel = e < vis && ((rk.sp_bits[sp_base + tj0 + (e < vis ? e : 0)] >> t) & 1u);
          sacc[i] = sel ? sacc[i] : -INFINITY;
        }
      } else if (__builtin_amdgcn_ballot_w64(vis < kTile || vlo > 0) != 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = tok_of(i) < vis && tok_of(i) >= vlo ? sacc[i] : -INFINITY;
      }
      mx = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[4], sacc[5]), fmaxf(sacc[6], sacc[7])));
    } else if (part == 1) {
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[8], sacc[9]), fmaxf(sacc[10], sacc[11])));
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[12], sacc[13]), fmaxf(sacc[14], sacc[15])));
      mx = fmaxf(mx, other_half(mx)) * c2;               // tile max in base-2 units
      const float m_new = fmaxf(m_run, mx);
      const bool move = m_new > m_run + 8.0f;             // move the reference only on a large jump
      const bool any_move = __builtin_amdgcn_ballot_w64(move) != 0;
      if (any_move) {
        const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        if (half == 0) reinterpret_cast<float*>(smem + kAlphaOff)[sbuf * kMaxRB * 32 + wave * 32 + n] = alpha;
        l_run *= alpha;
        if (move) m_run = m_new;
      }
      if (lane == 0) reinterpret_cast<uint8_t*>(smem + kFlagOff)[sbuf * 16 + wave] = any_move ? 1 : 0;
      neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
      psum = 0.f;
    } else if (part < kParts - 1) {
      const int i0 = 2 * (part - 2);
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c2, neg_m));
        psum += e;
        pk[i >> 3][i & 7] = (__bf16)e;
      }
    } else {
      l_run += psum;
    }
  };
  // Softmax of one whole tile (split-role waves).  After the chunk's first
  // tile every row that sees the whole tile has a finite reference within 2^8
  // of its running max, so such a tile is first weighted against the current
  // reference: when no lane's sum of weights exceeds 2^8 (every weight is
  // non-negative, so then none does) the reference need not move and the
  // tile max is never computed.  Otherwise -- an overflow, a larger max, many
  // large weights, or a tile that crosses some row's visible limit -- the
  // exact pieces above recompute it.
  auto softmax_tile = [&](bool first) {
    if (!first && !sparse_bits && __builtin_amdgcn_ballot_w64(vis < kTile || vlo > 0) == 0) {
      const float nm = -m_run;
      float e[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c2, nm));
      const float s = (((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]))) +
                      (((e[8] + e[9]) + (e[10] + e[11])) + ((e[12] + e[13]) + (e[14] + e[15])));
      if (__builtin_amdgcn_ballot_w64(!(s <= 256.0f)) == 0) {   // (also catches inf)
#pragma unroll
        for (int i = 0; i < 16; ++i) pk[i >> 3][i & 7] = (__bf16)e[i];
        if (lane == 0) reinterpret_cast<uint8_t*>(smem + kFlagOff)[sbuf * 16 + wave] = 0;
        l_run += s;
        return;
      }
    }
#pragma unroll
    for (int part = 0; part < kParts; ++part) softmax_part(part);
  };
  // P^T of this row block: k-step kk of lane half h at byte kk*32 + h*16
  auto write_p = [&](int buf) {
    *reinterpret_cast<bf16x8*>(p_addr(buf, wave * 32 + n, 0)) = pk[0];
    *reinterpret_cast<bf16x8*>(p_addr(buf, wave * 32 + n, 1)) = pk[1];
  };

  // Rescale this wave's columns of the row blocks whose reference moved.
  auto rescale = [&](int buf) {
    const uint32_t flags = *reinterpret_cast<const uint32_t*>(smem + kFlagOff + buf * 16);
    const uint32_t fu = __builtin_amdgcn_readfirstlane(flags);
    if (fu != 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if ((fu >> (8 * rb)) & 0xff) {
          const float alpha = reinterpret_cast<const float*>(smem + kAlphaOff)[buf * kMaxRB * 32 + rb * 32 + n];
#pragma unroll
          for (int cb = 0; cb < kWaveCols; ++cb) oacc[rb][cb] *= alpha;
        }
      }
    }
  };

  // O^T += V^T P^T for the tile in stage `st`: this wave's 4 column blocks x
  // RB row blocks x 2 k-steps, V^T fragments by transpose reads (kPvAhead
  // ahead), P^T fragments of a k-step read half a k-step ahead.
  auto pv = [&](const char* st, int pbuf) {
    const char* vb = st + v_off;
    bf16x8 pf[RB][2];
    auto read_p = [&](int kk) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) pf[rb][kk] = *reinterpret_cast<const bf16x8*>(p_addr(pbuf, rb * 32 + n, kk));
    };
    read_p(0);
    constexpr int kFrags = 2 * kWaveCols;             // (k-step, column block) pairs
    auto vfrag = [&](int f) {
      const int kk = f / kWaveCols, cb = f % kWaveCols;
      const char* a = vb + kk * (16 * kRowSlots * 16) + cb * 64;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 2 * kRowSlots * 16));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int kAhead = kPvAhead;
    bf16x8 vf[kFrags];
#pragma unroll
    for (int f = 0; f < kAhead && f < kFrags; ++f) vf[f] = vfrag(f);
#pragma unroll
    for (int f = 0; f < kFrags; ++f) {
      if (f + kAhead < kFrags) vf[f + kAhead] = vfrag(f + kAhead);
      if (f == kWaveCols / 2) read_p(1);
      const int kk = f / kWaveCols, cb = f % kWaveCols;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        oacc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[f], pf[rb][kk], oacc[rb][cb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // next tile's loads: the general path now, the fast path returned for the caller
  auto start_tile_loads = [&](int nt, const char*& ntb, uint32_t& nlds) -> bool {
    const bool fast = tile_is_fast(nt);
    ntb = fast ? tile_base_of(nt) : nullptr;
    if (nt < ntiles && (!fast || ntb == nullptr)) load_tile_general(nt);
    nlds = lds0 + (nt % kStages) * kStageBytes;
    return fast && ntb != nullptr;
  };

  {
    // ---- split roles.  Every role passes the same barriers: one before the
    // loop (tile 0 landed) and one per tile (A: tile it+1 landed, every wave
    // done with tile it-1, P^T and factors of tile it visible).
    // Issue priority: the loader first (its loads keep HBM busy), then the
    // score/softmax waves (they produce P, the PV waves' input), then PV.
    if (qk_wave) {
      __builtin_amdgcn_s_setprio(2);
      load_q();
      if (ntiles > 0) {
        wait_tiles_then_barrier<kMyLoads>(0);
        sacc = qk(smem);
        cap(sacc, row_lo);
        vis = lim - row_lo;
        tj0 = row_lo;
        vlo = low - row_lo;
        sbuf = 0;
        softmax_tile(true);
        write_p(0);
#pragma unroll 1
        for (int it = 0; it < ntiles; ++it) {
          wait_tiles_then_barrier<kMyLoads>(0);
          if (it + 1 < ntiles) {
            sacc = qk(smem + ((it + 1) % kStages) * kStageBytes);
            cap(sacc, row_lo + (it + 1) * kTile);
            vis = lim - (row_lo + (it + 1) * kTile);
            tj0 = row_lo + (it + 1) * kTile;
            vlo = low - (row_lo + (it + 1) * kTile);
            sbuf = (it + 1) & 1;
            softmax_tile(false);
            write_p((it + 1) & 1);
          }
        }
      }
    } else if (pv_wave) {
      init_o();
      if (ntiles > 0) {
        wait_tiles_then_barrier<kMyLoads>(0);
#pragma unroll 1
        for (int it = 0; it < ntiles; ++it) {
          wait_tiles_then_barrier<kMyLoads>(0);
          rescale(it & 1);
          pv(smem + (it % kStages) * kStageBytes, it & 1);
        }
      }
    } else {
      // the loader (and, with fewer than 3 row blocks, idle waves); only
      // this wave reads the page table, so the others start their own loads
      // without waiting for it
      __builtin_amdgcn_s_setprio(3);
      if (kAligned) load_page_table(pt_base);
      // the per-lane byte offsets of a fast tile's loads are the same for
      // every tile: computed once, kept in registers
      uint32_t foff[kMyLoads];
#pragma unroll
      for (int k = 0; k < kMyLoads; ++k) foff[k] = fast_offset(k);
      auto issue_fast_tile = [&](const char* tb, uint32_t lds_stage) {
        if (!loads_here) return;
#pragma unroll
        for (int k = 0; k < kMyLoads; ++k) dma16_sbase(tb, foff[k], lds_stage + (uint32_t)(load_slot0(k) * 16));
      };
#pragma unroll 1
      for (int it = 0; it < kStages - 1 && it < ntiles; ++it) {
        const char* tb = tile_is_fast(it) ? tile_base_of(it) : nullptr;
        if (tb) issue_fast_tile(tb, lds0 + (it % kStages) * kStageBytes);
        else load_tile_general(it);
      }
      if (ntiles > 0) {
        wait_tiles_then_barrier<kMyLoads>(ntiles - 1 < 2 ? ntiles - 1 : 2);
#pragma unroll 1
        for (int it = 0; it < ntiles; ++it) {
          wait_tiles_then_barrier<kMyLoads>(it + 2 < ntiles ? 1 : 0);
          const char* ntb;
          uint32_t nlds;
          if (start_tile_loads(it + kStages - 1, ntb, nlds)) issue_fast_tile(ntb, nlds);
        }
      }
    }
  }
  // every load has landed by now; make that explicit before the LDS is reused
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: QK waves publish 1 / l of their rows and store lse; every
  // wave normalises and stores its columns
  float* const inv_lds = reinterpret_cast<float*>(smem + kInvOff);
  if (qk_wave) {
    const float l_tot = l_run + other_half(l_run);
    float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    float lse2 = l_tot > 0.f ? m_run + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    if (rk.sinks != nullptr && wi.k == 0 && valid) {
      // the sink's term 2^sg joins the denominator of the request's first
      // chunk, against a reference that covers both
      const float sg = rk.sinks[R % p.H] * kLog2e;
      if (sg > -INFINITY) {
        const float ref = l_tot > 0.f ? fmaxf(m_run, sg) : sg;
        const float a = l_tot > 0.f ? __builtin_amdgcn_exp2f(m_run - ref) : 0.f;
        const float lt = l_tot * a + __builtin_amdgcn_exp2f(sg - ref);
        inv = a / lt;
        lse2 = ref + __builtin_amdgcn_logf(lt);
      }
    }
    if (half == 0) {
      inv_lds[wave * 32 + n] = inv;
      if (valid) {
        const float lse_out = p.out_base2 ? lse2 : lse2 * kLn2;
        if (!direct) p.ws_lse[part_slot(p, chunk) * p.M + R] = lse2;
        else if (p.records) rk.rec[rec_index(p, p.partials > 0 ? wi.k : 0, b, R) * (kDV / 4 + 1) + kDV / 4] =
            make_uint2(__float_as_uint(lse_out), 0u);
        else rk.lse[out_row0 + R] = lse_out;
      }
    }
  }
  lds_barrier();
  if (!pv_wave) return;
  // a request's only chunk (or an unmerged part) stores o itself in fp32; the
  // chunks of a request with several store their partial o as bf16 (rounded
  // to nearest even), merged by the chunk combine
  float* const out_base = direct && !p.records && !p.o_bf16 ? rk.o + out_row0 * kDV + cgrp * kWaveCols * 32 : nullptr;
  uint16_t* const out16_base =
      direct && p.o_bf16 ? reinterpret_cast<uint16_t*>(rk.o) + out_row0 * kDV + cgrp * kWaveCols * 32 : nullptr;
  uint2* const rec_base = direct && p.records ? rk.rec + cgrp * kWaveCols * 8 : nullptr;
  const int32_t rec_part = p.partials > 0 ? wi.k : 0;
  uint16_t* const part_base = direct ? nullptr : p.ws_o + part_slot(p, chunk) * p.M * kDV + cgrp * kWaveCols * 32;
  {
    // Normalise and store this wave's 128 columns of each row block.  The
    // accumulator layout gives a lane 16-byte pieces of 4 different 128-byte
    // lines per row; staging the block through this wave's own slice of the
    // (now idle) tile ring turns the stores into 512-byte row segments.
    float* const stage = reinterpret_cast<float*>(smem + cgrp * kEpiWaveBytes);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float inv = inv_lds[rb * 32 + n];
#pragma unroll
      for (int cb = 0; cb < kWaveCols; ++cb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float4 v;
          v.x = oacc[rb][cb][4 * q4 + 0] * inv;
          v.y = oacc[rb][cb][4 * q4 + 1] * inv;
          v.z = oacc[rb][cb][4 * q4 + 2] * inv;
          v.w = oacc[rb][cb][4 * q4 + 3] * inv;
          *reinterpret_cast<float4*>(stage + n * kEpiPitch + cb * 32 + 8 * q4 + 4 * half) = v;
        }
      }
      lds_wait();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 2 * i + half;
        const float4 v = *reinterpret_cast<const float4*>(stage + r * kEpiPitch + 4 * n);
        const int Rr = row0 + rb * 32 + r;
        if (Rr < p.M) {
          typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
          typedef float f32x4_t __attribute__((ext_vector_type(4)));
          if (direct && p.o_bf16) {
            // o in bf16, 4 values (round to nearest even) per 8-byte store
            const bf16x4_t h = __builtin_convertvector((f32x4_t){v.x, v.y, v.z, v.w}, bf16x4_t);
            *reinterpret_cast<bf16x4_t*>(out16_base + (int64_t)Rr * kDV + 4 * n) = h;
          } else if (direct && !p.records) {
            *reinterpret_cast<float4*>(out_base + (int64_t)Rr * kDV + 4 * n) = v;
          } else if (direct) {
            // packed record: 4 bf16 (round to nearest even) per 8-byte unit
            const bf16x4_t h = __builtin_convertvector((f32x4_t){v.x, v.y, v.z, v.w}, bf16x4_t);
            rec_base[rec_index(p, rec_part, b, Rr) * (kDV / 4 + 1) + n] = __builtin_bit_cast(uint2, h);
          } else {
            const bf16x4_t h = __builtin_convertvector((f32x4_t){v.x, v.y, v.z, v.w}, bf16x4_t);
            *reinterpret_cast<bf16x4_t*>(part_base + (int64_t)Rr * kDV + 4 * n) = h;
          }
        }
      }
      lds_wait();   // the next block overwrites the slice
    }
  }
}

struct Plan {
  int RB, mgroups;
  int64_t Bv;              // requests of all ranks in the launch
  int64_t slots;           // chunk slots; the grid has slots * mgroups workgroups
  int32_t forced, target;  // Params::forced_splits, Params::target_chunks
  bool combine;            // some request may have several chunks
  size_t ws_bytes, table_off;
};

// Checks of one rank's arguments (pointers are not read).
int check_args(const dcp_attn_args* a) {
  if (a == nullptr) return DCP_EINVAL;
  if (!layout_ok(a->layout)) return DCP_EINVAL;
  if (a->rank < 0 || a->rank >= a->layout.n_stripes) return DCP_EINVAL;
  if (a->batch < 1 || a->q_len < 1 || a->n_heads < 1) return DCP_EINVAL;
  if (a->head_dim != kD || a->v_dim != kDV) return DCP_EUNSUPPORTED;
  if (a->bt_cols < 1 || a->num_pages < 1) return DCP_EINVAL;
  if (a->lse_base != 0 && a->lse_base != 1) return DCP_EINVAL;
  if (a->num_splits < 0) return DCP_EINVAL;
  if (a->partials != 0 && (a->partials != 1 || a->num_splits < 1)) return DCP_EINVAL;
  if (a->window < 0 || !(a->softcap >= 0.f) || a->softcap == INFINITY) return DCP_EINVAL;
  if (a->out_records != 0 && a->out_records != 1) return DCP_EINVAL;
  if (a->out_records && a->n_heads % a->layout.n_stripes != 0) return DCP_EINVAL;
  if (a->o_bf16 != 0 && (a->o_bf16 != 1 || a->out_records)) return DCP_EINVAL;
  if ((a->softcap > 0.f || a->bias_slopes != nullptr) && !(a->scale > 0.f)) return DCP_EINVAL;
  if (a->sparse_rows != nullptr) {
    if (a->sparse_bits == nullptr || a->sparse_count == nullptr || a->sparse_stride < 1) return DCP_EINVAL;
    if (a->window > 0 || a->bias_slopes != nullptr) return DCP_EUNSUPPORTED;   // positions are not tracked
    if (a->q_len > 32) return DCP_EUNSUPPORTED;                                // one selection bit per draft
  }
  const int64_t M = (int64_t)a->q_len * a->n_heads;
  const int64_t max_rows = a->sparse_rows ? (int64_t)a->sparse_stride : (int64_t)a->bt_cols * a->layout.page_size;
  if (M > (1 << 20) || max_rows > 0x7fffffff - 64) return DCP_EUNSUPPORTED;
  if ((int64_t)a->layout.n_stripes * a->layout.interleave > 0x7fffffff) return DCP_EUNSUPPORTED;
  return DCP_OK;
}

// The ranks of one launch share everything but the rank's own data (pool,
// table, outputs, sink, selection).
bool same_launch(const dcp_attn_args& a, const dcp_attn_args& b) {
  return a.layout.n_stripes == b.layout.n_stripes && a.layout.interleave == b.layout.interleave &&
         a.layout.page_size == b.layout.page_size && a.batch == b.batch && a.q_len == b.q_len &&
         a.n_heads == b.n_heads && a.q == b.q && a.seq_len == b.seq_len && a.scale == b.scale &&
         a.lse_base == b.lse_base && a.num_splits == b.num_splits && a.window == b.window &&
         a.softcap == b.softcap && a.partials == b.partials && a.bias_slopes == b.bias_slopes &&
         a.out_records == b.out_records && a.o_bf16 == b.o_bf16 &&
         (a.sparse_rows == nullptr) == (b.sparse_rows == nullptr);
}

// a * b for a, b >= 0, or INT64_MAX when the product does not fit
int64_t mul_or_max(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

int make_plan(const dcp_attn_args* args, int32_t n, Plan* pl) {
  if (args == nullptr || pl == nullptr || n < 1) return DCP_EINVAL;
  if (n > kMaxRanks) return DCP_EUNSUPPORTED;
  for (int32_t i = 0; i < n; ++i) {
    const int rc = check_args(&args[i]);
    if (rc != DCP_OK) return rc;
    if (!same_launch(args[0], args[i])) return DCP_EINVAL;
  }
  const dcp_attn_args* a = &args[0];
  const int64_t M = (int64_t)a->q_len * a->n_heads;
  int64_t max_rows = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t m = args[i].sparse_rows ? (int64_t)args[i].sparse_stride
                                          : (int64_t)args[i].bt_cols * args[i].layout.page_size;
    max_rows = m > max_rows ? m : max_rows;
  }
  // the kernel indexes query rows and workgroups in 32 bits
  if (M > 0x7fffffff) return DCP_EUNSUPPORTED;
  pl->Bv = (int64_t)n * a->batch;
  // query rows per workgroup: up to 3 blocks of 32; above 96 rows the rows
  // are cut into groups (the workgroups of one group run side by side on
  // one XCD and share each KV tile through its L2), with the block count
  // that pads the fewest rows
  if (M <= 32 * kMaxRB) {
    pl->RB = (int)ceil_div(M, 32);
  } else {
    pl->RB = kMaxRB;
    for (int rb = kMaxRB - 1; rb >= 1; --rb)
      if (ceil_div(M, 32 * rb) * 32 * rb < ceil_div(M, 32 * pl->RB) * 32 * pl->RB) pl->RB = rb;
  }
  pl->mgroups = (int)ceil_div(M, 32 * pl->RB);
  const int64_t tiles_max = ceil_div(max_rows, kTile);
  if (a->partials) {
    // unmerged parts: exactly num_splits per request, some possibly empty
    pl->forced = a->num_splits;
    pl->target = 0;
    pl->slots = mul_or_max(pl->Bv, a->num_splits);
  } else if (a->num_splits > 0) {
    // a fixed number of chunks per request
    pl->forced = (int32_t)(a->num_splits < tiles_max ? a->num_splits : tiles_max);
    pl->target = 0;
    pl->slots = mul_or_max(pl->Bv, pl->forced);
  } else {
    // balanced chunks: one workgroup per compute unit, in one round when the
    // requests are fewer than the compute units; otherwise chunks of the mean
    // per-unit share (at most target + requests of them)
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
      int v = 0;
      if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    pl->forced = 0;
    pl->target = cus / pl->mgroups > 1 ? cus / pl->mgroups : 1;
    pl->slots = pl->target > pl->Bv ? pl->target : pl->target + pl->Bv;
    if (pl->target <= pl->Bv && pl->mgroups > 1) {
      // chunks capped at kGroupChunkTiles tiles: at most that share of every request, plus one
      const int64_t capped = mul_or_max(pl->Bv, ceil_div(tiles_max, kGroupChunkTiles) + 1);
      pl->slots = capped > pl->slots ? capped : pl->slots;
    }
  }
  // a multiple of 8 * kChunkGroup slots: the kernel's block order hands
  // groups of kChunkGroup chunks to the 8 XCDs in turn
  if (pl->slots > 0x7fffffff) return DCP_EUNSUPPORTED;
  pl->slots = ceil_div(pl->slots, 8 * kChunkGroup) * 8 * kChunkGroup;
  if (mul_or_max(pl->slots, pl->mgroups) > 0x7fffffff || pl->Bv > 0x7fffffff / 2) return DCP_EUNSUPPORTED;
  pl->combine = pl->forced != 1 && !a->partials;
  // chunk partials (o, base-2 lse) and the chunk table
  if (pl->combine) {
    const size_t part = (size_t)pl->slots * M * (kDV * sizeof(uint16_t) + sizeof(float));
    pl->table_off = (part + 255) & ~(size_t)255;
    pl->ws_bytes = pl->table_off + (size_t)2 * pl->Bv * sizeof(int32_t);
  } else {
    pl->table_off = 0;
    pl->ws_bytes = 0;
  }
  return DCP_OK;
}

// Merge of each request's chunks (one wavefront per output row, 16-byte
// loads of the bf16 partials, 8 chunks in flight at once): requests cut
// into one chunk were written by the attention kernel itself and are left
// alone; the chunks partition the request's rows, so their partials merge
// exactly like stripes (base-2 partial lse).
constexpr int kCombineWaves = 4;       // wavefronts per block, one output row each
constexpr int kCombineGroup = 8;       // chunk partials loaded at once

__global__ void __launch_bounds__(64 * kCombineWaves) chunk_combine_kernel(Params p) {
  int64_t bid = blockIdx.x;
  if ((gridDim.x & 7) == 0) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
  const int lane = threadIdx.x & 63;
  const int64_t Bv = (int64_t)p.nr * p.B;
  const int64_t row = bid * kCombineWaves + (threadIdx.x >> 6);
  if (row >= Bv * p.M) return;
  const int32_t v = (int32_t)(row / p.M), m = (int32_t)(row - (int64_t)v * p.M);
  const int32_t n = p.table[v];
  if (n <= 1) return;                        // one chunk: written by the attention kernel
  const int64_t c0 = p.table[Bv + v];
  if (c0 < 0 || c0 + n > p.slots) return;   // (never written so: entries are cut to the slots)
  const int32_t ri = v / p.B, b = v - ri * p.B;
  const RankPtrs& rk = p.rk[ri];
  const int64_t out = (int64_t)b * p.M + m;
  constexpr int v4 = kDV / 4;
  // lane l takes values 8l .. 8l+7 (16 bytes of bf16) of each part,
  // kCombineGroup parts in flight at once; the lse of parts r0 .. r0+63 sit
  // one per lane (base 2).  The first group's loads go out with the lse's.
  // part k of the request sits in workspace slot part_slot(c0 + k)
  const float* const lse0 = p.ws_lse + m;
  const uint4* const part0 = reinterpret_cast<const uint4*>(p.ws_o + (int64_t)m * kDV) + lane;
  const int64_t part_stride = p.M * (kDV / 8);
  auto lse_of = [&](int32_t k) { return lse0[part_slot(p, c0 + k) * p.M]; };
  auto part_of = [&](int32_t k) { return part0[part_slot(p, c0 + k) * part_stride]; };
  float lp = lane < n ? lse_of(lane) : -INFINITY;
  uint4 x[kCombineGroup];
#pragma unroll
  for (int k = 0; k < kCombineGroup; ++k)
    x[k] = k < n ? part_of(k) : make_uint4(0u, 0u, 0u, 0u);
  float mx = lp;
  for (int r0 = 64; r0 < n; r0 += 64)
    if (r0 + lane < n) mx = fmaxf(mx, lse_of(r0 + lane));
  mx = wave_max(mx);
  // the exact merge: weights 2^(lse_k - max) / sum; parts of weight zero are
  // selected away, whatever they hold
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse_out = -INFINITY;
  if (mx != -INFINITY) {
    float wsum = lp == -INFINITY ? 0.f : exp2f(lp - mx);
    for (int r0 = 64; r0 < n; r0 += 64) {
      const float l = r0 + lane < n ? lse_of(r0 + lane) : -INFINITY;
      wsum += l == -INFINITY ? 0.f : exp2f(l - mx);
    }
    wsum = wave_sum(wsum);
    const float inv = 1.0f / wsum;
    float w = lp == -INFINITY ? 0.f : exp2f(lp - mx) * inv;   // lane k: weight of part r0 + k
    for (int g = 0; g < n; g += kCombineGroup) {
      if (g > 0) {
        if ((g & 63) == 0) {
          lp = g + lane < n ? lse_of(g + lane) : -INFINITY;
          w = lp == -INFINITY ? 0.f : exp2f(lp - mx) * inv;
        }
#pragma unroll
        for (int k = 0; k < kCombineGroup; ++k)
          x[k] = g + k < n ? part_of(g + k) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int k = 0; k < kCombineGroup; ++k) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), (g + k) & 63));
        if (g + k < n && wk != 0.f) {
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
    lse_out = p.out_base2 ? mx + lw2 : (mx + lw2) * kLn2;
  }
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  if (p.o_bf16) {
    // o_r in bf16 (one 16-byte store per lane), lse in float32
    const bf16x4_t h0 = __builtin_convertvector((f32x4_t){acc[0], acc[1], acc[2], acc[3]}, bf16x4_t);
    const bf16x4_t h1 = __builtin_convertvector((f32x4_t){acc[4], acc[5], acc[6], acc[7]}, bf16x4_t);
    uint4* const o16 = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(rk.o) + out * kDV);
    const uint2 a0 = __builtin_bit_cast(uint2, h0), a1 = __builtin_bit_cast(uint2, h1);
    o16[lane] = make_uint4(a0.x, a0.y, a1.x, a1.y);
    if (lane == 0) rk.lse[out] = lse_out;
  } else if (p.records) {
    uint2* const rec = rk.rec + rec_index(p, 0, b, m) * (v4 + 1);
    const bf16x4_t h0 = __builtin_convertvector((f32x4_t){acc[0], acc[1], acc[2], acc[3]}, bf16x4_t);
    const bf16x4_t h1 = __builtin_convertvector((f32x4_t){acc[4], acc[5], acc[6], acc[7]}, bf16x4_t);
    rec[2 * lane] = __builtin_bit_cast(uint2, h0);
    rec[2 * lane + 1] = __builtin_bit_cast(uint2, h1);
    if (lane == 0) rec[v4] = make_uint2(__float_as_uint(lse_out), 0u);
  } else {
    float4* const o = reinterpret_cast<float4*>(rk.o) + out * v4;
    o[2 * lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    o[2 * lane + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    if (lane == 0) rk.lse[out] = lse_out;
  }
}

template <int RB, bool kLogit>
int launch(const Params& prm, int64_t blocks, hipStream_t stream) {
  if (prm.P % kTile == 0)
    hipLaunchKernelGGL((stripe_attn_kernel<RB, true, kLogit>), dim3((unsigned)blocks), dim3(64 * kNW), 0, stream, prm);
  else
    hipLaunchKernelGGL((stripe_attn_kernel<RB, false, kLogit>), dim3((unsigned)blocks), dim3(64 * kNW), 0, stream, prm);
  return launch_status();
}

template <int RB>
int launch(const Params& prm, int64_t blocks, hipStream_t stream) {
  const bool logit = prm.cap_out > 0.f || prm.slopes != nullptr;
  return logit ? launch<RB, true>(prm, blocks, stream) : launch<RB, false>(prm, blocks, stream);
}

// One launch (plus the chunk combine when a request has several chunks) for
// the n ranks of `args`; the workspace of args[0] serves them all.
int run(const dcp_attn_args* args, int32_t n, void* stream) {
  Plan pl;
  const int rc = make_plan(args, n, &pl);
  if (rc != DCP_OK) return rc;
  const dcp_attn_args* a = &args[0];
  for (int32_t i = 0; i < n; ++i) {
    const dcp_attn_args& x = args[i];
    if (x.q == nullptr || x.pool == nullptr || x.block_table == nullptr || x.seq_len == nullptr ||
        x.o == nullptr || (x.lse == nullptr && !x.out_records))
      return DCP_EINVAL;
  }
  if (pl.ws_bytes > 0 && (a->workspace == nullptr || a->workspace_bytes < pl.ws_bytes)) return DCP_EINVAL;
  const int64_t M = (int64_t)a->q_len * a->n_heads;
  Params prm = {};
  prm.N = a->layout.n_stripes;
  prm.I = a->layout.interleave;
  prm.P = a->layout.page_size;
  prm.nr = n;
  prm.B = a->batch;
  prm.q_len = a->q_len;
  prm.H = a->n_heads;
  prm.M = (int32_t)M;
  prm.RB = pl.RB;
  prm.mgroups = pl.mgroups;
  prm.slots = (int32_t)pl.slots;
  prm.forced_splits = pl.forced;
  prm.partials = a->partials ? a->num_splits : 0;
  prm.target_chunks = pl.target;
  prm.q = (const __bf16*)a->q;
  prm.seq_len = a->seq_len;
  prm.c2 = a->scale * kLog2e;
  prm.window = a->window;
  prm.cap_in = a->softcap > 0.f ? a->scale / a->softcap : 0.f;
  prm.cap_out = a->softcap > 0.f ? a->softcap / a->scale : 0.f;
  prm.slopes = a->bias_slopes;
  prm.sparse = a->sparse_rows != nullptr;
  prm.inv_scale = a->scale > 0.f ? 1.0f / a->scale : 0.f;
  prm.out_base2 = a->lse_base;
  prm.records = a->out_records;
  prm.o_bf16 = a->o_bf16;
  prm.ws_o = pl.combine ? (uint16_t*)a->workspace : nullptr;
  prm.ws_lse = pl.combine ? reinterpret_cast<float*>(prm.ws_o + (size_t)pl.slots * M * kDV) : nullptr;
  prm.table = pl.combine ? (int32_t*)((char*)a->workspace + pl.table_off) : nullptr;
  prm.status = a->status;
  for (int32_t i = 0; i < n; ++i) {
    const dcp_attn_args& x = args[i];
    RankPtrs& r = prm.rk[i];
    r.pool = (const char*)x.pool;
    r.bt = x.block_table;
    r.o = x.out_records ? nullptr : x.o;
    r.lse = x.out_records ? nullptr : x.lse;
    r.rec = x.out_records ? reinterpret_cast<uint2*>(x.o) : nullptr;
    r.sinks = x.sinks;
    r.sp_rows = x.sparse_rows;
    r.sp_bits = x.sparse_bits;
    r.sp_count = x.sparse_count;
    r.num_pages = x.num_pages;
    r.rank = x.rank;
    r.bt_cols = x.bt_cols;
    r.sp_stride = x.sparse_stride;
  }
  const int64_t blocks = pl.slots * pl.mgroups;
  hipStream_t s = (hipStream_t)stream;
  int r;
  switch (pl.RB) {
    case 1: r = launch<1>(prm, blocks, s); break;
    case 2: r = launch<2>(prm, blocks, s); break;
    default: r = launch<3>(prm, blocks, s); break;
  }
  if (r != DCP_OK || !pl.combine) return r;
  const int64_t rows = pl.Bv * M;
  hipLaunchKernelGGL(chunk_combine_kernel, dim3((unsigned)ceil_div(rows, kCombineWaves)),
                     dim3(64 * kCombineWaves), 0, s, prm);
  return launch_status();
}

}  // namespace attn
}  // namespace dcp

using namespace dcp;
using namespace dcp::attn;

extern "C" int dcp_stripe_attn_workspace(const dcp_attn_args* args, size_t* bytes) {
  return dcp_stripe_attn_multi_workspace(args, 1, bytes);
}

extern "C" int dcp_stripe_attn(const dcp_attn_args* a, void* stream) { return run(a, 1, stream); }

extern "C" int dcp_stripe_attn_multi_workspace(const dcp_attn_args* args, int32_t n, size_t* bytes) {
  if (bytes == nullptr) return DCP_EINVAL;
  Plan pl;
  const int rc = make_plan(args, n, &pl);
  if (rc != DCP_OK) return rc;
  *bytes = pl.ws_bytes;
  return DCP_OK;
}

extern "C" int dcp_stripe_attn_multi(const dcp_attn_args* args, int32_t n, void* stream) {
  return run(args, n, stream);
}

// ---- dcp_stripe_attn_noalloc: the same call with a fixed scratch buffer in
// place of the caller's workspace, for callers that cannot allocate.  The
// buffer is a file-scope device array: each GPU the library's kernels load on
// holds its own copy (kNoAllocScratchBytes) until the process ends.  Host code
// never uses the array's name as an address: its device address is looked up
// once per device with hipGetSymbolAddress and kept.
namespace {
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kNoAllocMaxDevices = 64;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};

// device address of this device's copy of `scratch` (nullptr on a HIP error)
void* scratch_address(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" size_t dcp_stripe_attn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int dcp_stripe_attn_noalloc(const dcp_attn_args* args, void* stream) {
  Plan pl;
  const int rc = make_plan(args, 1, &pl);
  if (rc != DCP_OK) return rc;
  if (pl.ws_bytes > kNoAllocScratchBytes) return DCP_ESCRATCH;
  dcp_attn_args a = *args;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  if (pl.ws_bytes > 0) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return DCP_EHIP;
    void* ptr = scratch_address(dev);
    if (ptr == nullptr) return DCP_EHIP;
    a.workspace = ptr;
    a.workspace_bytes = kNoAllocScratchBytes;
  }
  return run(&a, 1, stream);
}
