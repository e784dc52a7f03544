/*
 * dcp.h -- C ABI of the MI355X (gfx950) decode-context-parallel (DCP) MLA
 * attention library, libdcp.so.
 *
 * DCP stripes the shared latent KV of absorbed MLA over N ranks by token
 * position: rank r stores the positions it owns compactly, each rank attends
 * all H query heads to its own stripe and returns a locally normalised output
 * with its log-sum-exp, and an exact LSE merge recombines the stripes
 * (page "DCP" (zdszero), "core abstraction" and "theory"; SGLang DCP docs,
 * "MLA decode dataflow").  On one GPU the N stripes are N separate pools and
 * every rank's kernel runs at its real per-rank shape.
 *
 * Conventions shared by every entry point:
 *  - Pointers named as device pointers must point to device memory (or
 *    memory the device can read/write); the caller owns all buffers.  The
 *    library never allocates or frees memory and keeps no state between calls,
 *    except the fixed scratch buffer of dcp_stripe_attn_noalloc (one per GPU,
 *    held until the process ends).
 *  - bfloat16 data is passed as raw 16-bit storage (void*).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues kernel launches on `stream` and returns; nothing is
 *    synchronised, and no call copies or clears memory with a runtime call,
 *    so a sequence of calls can be captured into a HIP graph and replayed.
 *  - Return value: DCP_OK, or a negative error code.  On any error return
 *    nothing has been enqueued.  Argument errors (DCP_EINVAL,
 *    DCP_EUNSUPPORTED) are detected on the host before any HIP call.
 *  - Errors that depend on device data (a page id outside the pool, a page
 *    table with no entry for a needed row, a negative position) cannot be seen
 *    on the host: the kernels then skip the offending row, never touch memory
 *    outside the buffers, and store DCP_ERANGE into *status when `status` is
 *    not NULL.  Kernels only ever store DCP_ERANGE there; the caller clears
 *    *status to DCP_OK beforehand.
 */
#ifndef DCP_H
#define DCP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCP_OK 0
#define DCP_EINVAL (-1)        /* invalid argument (NULL, negative size, bad layout) */
#define DCP_EUNSUPPORTED (-2)  /* shape outside what the kernels are built for */
#define DCP_EHIP (-3)          /* a HIP call or kernel launch failed */
#define DCP_ERANGE (-4)        /* device data out of range (stored into *status) */
#define DCP_ESCRATCH (-5)      /* needs more scratch than dcp_stripe_attn_noalloc's fixed buffer */

/* Token-to-rank layout.
 * n_stripes  N >= 1: DCP size (number of stripes / ranks).
 * interleave I >= 1: tokens are handed out in consecutive runs of I, one run
 *            per rank in turn (I = 1: token round robin, owner = p mod N;
 *            page "PCP/DCP" (obnotes) sections 5 and 6; vLLM-Ascend CP design,
 *            "block table", cp_kv_cache_interleave_size).
 * page_size  P >= 1, with P % I == 0 (the vLLM-Ascend design requires the
 *            block size to be a multiple of the interleave) or I % P == 0
 *            (a run of I tokens fills whole pages: page "PCP/DCP" (obnotes)
 *            section 6 lets the block be k physical pages).
 * For a global position p:
 *   owner(p) = floor(p / I) mod N
 *   row(p)   = floor(p / (I*N)) * I + p mod I          (compact local row)
 *   count_r(x) = #{ p in [0, x) : owner(p) = r }
 * and a local row j of rank r holds global position
 *   p = floor(j / I) * I * N + r * I + j mod I. */
typedef struct dcp_layout {
  int32_t n_stripes;
  int32_t interleave;
  int32_t page_size;
} dcp_layout;

/* Human-readable name of a return code (static storage, never NULL). */
const char* dcp_strerror(int code);

/* Library ABI version (incremented when a signature changes). */
int dcp_abi_version(void);

/* dcp_slot_map -- owner, local row and physical slot of n positions.
 * Page "DCP": ownership is a pure function of the position; page "PCP/DCP",
 * "KV cache management": slot = page_id * page_size + offset in page, the page
 * id coming from the request's page table.
 *
 * pos   [n] int64  device, global positions (>= 0).
 * req   [n] int32  device, request index of each position, or NULL (all 0).
 * block_table [bt_rows][bt_cols] int32 device, rank `rank`'s page table:
 *       entry [b][k] is the page of this rank's pool holding local rows
 *       k*P .. k*P+P-1 of request b; -1 = none.  May be NULL (no slots).
 * owner [n] int32 out, row [n] int64 out, slot [n] int64 out: each may be NULL.
 *       slot[i] = -1 when rank < 0, block_table is NULL, or owner != rank.
 *       An owned position whose request or page-table column is out of range,
 *       or whose entry is negative, also gets -1 and raises DCP_ERANGE.
 *       A negative position gets owner = -1, row = -1, slot = -1, DCP_ERANGE.
 * status  device int32, nullable (see conventions). */
int dcp_slot_map(dcp_layout layout, int32_t rank,
                 const int64_t* pos, const int32_t* req, int64_t n,
                 const int32_t* block_table, int32_t bt_rows, int32_t bt_cols,
                 int32_t* owner, int64_t* row, int64_t* slot,
                 int32_t* status, void* stream);

/* dcp_local_count -- every rank's share of n intervals [start, start+len).
 * Page "DCP", idea one, and page "PCP/DCP" section 6: the share of rank r is
 * count_r(start + len) - count_r(start) with global positions; start = 0
 * gives the local length of a request of `len` tokens.
 * start [n] int64 device (NULL = all 0), len [n] int64 device (>= 0),
 * count [n][N] int64 device out.  Negative start/len: counts 0, DCP_ERANGE
 * is not reported (no status); the caller validates lengths. */
int dcp_local_count(dcp_layout layout, const int64_t* start, const int64_t* len,
                    int64_t n, int64_t* count, void* stream);

/* dcp_kv_write -- owner-filtered paged write of new latent rows.
 * Page "MLA 的 Decode Context Parallelism", section 4, stage 2: each new
 * 576-dim latent row is stored only on the rank that owns its position, at
 * its compact slot; rows of other ranks are skipped (not read).
 * kv_new [T][row_dim] bf16 device; row_dim % 8 == 0.
 * pos [T] int64, req [T] int32 (NULL = all 0) device.
 * block_table as in dcp_slot_map (required).
 * pool [num_pages][P][row_dim] bf16 device, this rank's pool.
 * A row whose page id is outside [0, num_pages) or whose table entry is
 * missing is skipped and raises DCP_ERANGE. */
int dcp_kv_write(dcp_layout layout, int32_t rank,
                 const void* kv_new, int32_t row_dim, int64_t T,
                 const int64_t* pos, const int32_t* req,
                 const int32_t* block_table, int32_t bt_rows, int32_t bt_cols,
                 void* pool, int64_t num_pages,
                 int32_t* status, void* stream);

/* dcp_relayout -- prefill (DCP1) to decode (DCP-N) token relayout.
 * Page "PCP/DCP" (obnotes), "PD + DCP: extracting this rank's tokens from
 * full source pages"; SGLang DCP docs, "DCP x PD disaggregation".  For each
 * request b the positions [start[b], start[b] + len[b]) that rank `rank`
 * owns -- chosen by the request's global position -- are copied from the
 * request's dense source pages (position t at source row t) to the rank's
 * compact pool (local row j at block_table[b][j / P] * P + j % P).  Exactly
 * count_r(start + len) - count_r(start) rows are moved per request, so rows
 * of a partly filled final source page never leak; nothing else is written.
 * row_dim           row length in bf16 (the same on both sides), % 8 == 0.
 * src_pool          [src_pages][src_page_size][row_dim] bf16 device.
 * src_block_table   [batch][src_bt_cols] int32 device: the request's source pages.
 * start, len        [batch] int64 device (start >= 0 and len >= 0, else the
 *                   request is skipped and DCP_ERANGE raised).
 * max_len           host int64, an upper bound of len used to size the launch
 *                   (a longer len is still moved completely, more slowly).
 * block_table, bt_cols, pool, num_pages  the rank's pool as in dcp_kv_write
 *                   (page size = layout.page_size).
 * A row whose source or destination page is missing or out of range is
 * skipped and raises DCP_ERANGE.  batch > 65535: DCP_EUNSUPPORTED. */
int dcp_relayout(dcp_layout layout, int32_t rank, int32_t row_dim,
                 const void* src_pool, int64_t src_pages, int32_t src_page_size,
                 const int32_t* src_block_table, int32_t src_bt_cols,
                 const int64_t* start, const int64_t* len, int32_t batch, int64_t max_len,
                 const int32_t* block_table, int32_t bt_cols,
                 void* pool, int64_t num_pages,
                 int32_t* status, void* stream);

/* Arguments of one rank's stripe attention (absorbed MLA decode).
 * Query row i of request b, query t, head h: q[b][t][h][0..575] =
 * [absorbed nope part (512) || rope part (64)] (page "MLA 的 DCP", section 2).
 * The key of a cached token is its whole 576-dim latent row, the value its
 * first v_dim = 512 dims.  The q_len queries of request b sit at global
 * positions seq_len[b] - q_len + t and see the cached positions p <= their
 * own (causal among drafts; SGLang DCP docs, "DCP x speculative decoding":
 * the kernel gets the global lengths and its rank).
 *
 * layout, rank  rank r's stripe under `layout` (0 <= rank < N).
 * batch, q_len, n_heads  B >= 1, q_len >= 1, H >= 1.
 * head_dim, v_dim        must be 576 and 512 (else DCP_EUNSUPPORTED).
 * q           [B][q_len][H][head_dim] bf16 device.
 * pool        [num_pages][P][head_dim] bf16 device, this rank's pool.
 * block_table [B][bt_cols] int32 device, this rank's page table.
 * seq_len     [B] int32 device, GLOBAL context lengths (>= q_len).
 * scale       softmax scale applied to q.k (e.g. 1/sqrt(192)).
 * lse_base    0: lse in natural log; 1: lse in log2 (same partition function,
 *             lse2 = lse * log2(e)); the output o does not depend on it.
 * num_splits  0: the library cuts every request's local rows into chunks
 *             of whole 32-token tiles balanced over the whole batch (ragged
 *             lengths included), one workgroup per chunk; k > 0: each
 *             request into k chunks of equal length (fewer when it is
 *             shorter than k tiles).
 * workspace, workspace_bytes  device scratch of at least the size
 *             dcp_stripe_attn_workspace() reports for these arguments (0 only
 *             for num_splits = 1).  It holds each chunk's partial (o as
 *             bfloat16, rounded to nearest even, and its lse as float32) and
 *             the chunk table; a second kernel on the same stream merges the
 *             chunks of every request that has more than one.  (A request
 *             cut into one chunk writes o_r directly, without the rounding.)  Its
 *             contents need no initialisation.  Calls that overlap in time
 *             must not share a workspace; with a workspace each, calls on
 *             different streams may run at the same time (the library keeps
 *             no other state between calls).
 * o    [B][q_len][H][v_dim] fp32 device out: o_r, normalised inside the stripe.
 * lse  [B][q_len][H] fp32 device out: lse_r in the chosen base.
 *      A query with no visible row in this stripe gets o = 0, lse = -inf
 *      (zero weight in the merge; page "PCP/DCP" section 4.1).
 * status device int32, nullable: DCP_ERANGE when a needed page id is outside
 *      [0, num_pages) or missing from the table (that request's output is
 *      then unspecified, memory outside the buffers is never read).
 *
 * Variants that keep the merge exact (page "DCP", conditions for merging:
 * a mask only shrinks the visible set, a sink is one extra logit term in one
 * shard, an elementwise logit transform couples no positions):
 * window   W > 0: a query at global position t sees t - W < p <= t (sliding
 *          window); 0: the whole context.  < 0: DCP_EINVAL.
 * softcap  c > 0: every scaled score s becomes c * tanh(s / c) before the
 *          softmax; 0: none.  Negative, NaN or inf: DCP_EINVAL.
 * sinks    [n_heads] fp32 device, nullable: a natural-log logit per head that
 *          joins the softmax denominator with value zero.  Pass it on
 *          exactly one rank's call: the merge adds the stripes' partition
 *          functions, so a sink given to k ranks counts k times.  A row with
 *          no visible position then gets o = 0 and lse = the sink.
 * bias_slopes [n_heads] fp32 device, nullable: linear position bias (ALiBi
 *          style) -- the logit of position p for a query at t of head h gains
 *          bias_slopes[h] * (p - t), natural-log units, after the softcap.
 *          Positions are global, so every rank passes the same slopes.
 * sparse_rows, sparse_bits, sparse_count, sparse_stride  nullable (all or
 *          none): a sparse selection from dcp_sparse_plan for this rank.  The
 *          stripe then attends, for each query token t, only to the entries
 *          whose bit t is set (the selected positions it owns), instead of
 *          its whole stripe.  With window > 0 or bias_slopes: DCP_EUNSUPPORTED. */
typedef struct dcp_attn_args {
  dcp_layout layout;
  int32_t rank;
  int32_t batch;
  int32_t q_len;
  int32_t n_heads;
  int32_t head_dim;
  int32_t v_dim;
  const void* q;
  const void* pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t bt_cols;
  const int32_t* seq_len;
  float scale;
  int32_t lse_base;
  int32_t num_splits;
  void* workspace;
  size_t workspace_bytes;
  float* o;
  float* lse;
  int32_t* status;
  int32_t window;
  float softcap;
  const float* sinks;
  int32_t partials;
  const float* bias_slopes;
  const int32_t* sparse_rows;
  const uint32_t* sparse_bits;
  const int32_t* sparse_count;
  int32_t sparse_stride;
  int32_t out_records;
  int32_t o_bf16;
} dcp_attn_args;

/* Unmerged parts (page "DCP", "unification with online softmax": the split
 * inside a stripe and the split across stripes are one merge, so both can be
 * folded into a single pass when o_r itself is not needed):
 * partials  0: o, lse are o_r, lse_r as above.  1 (needs num_splits = k >= 1):
 *           every request's stripe is cut into exactly k parts of
 *           ceil(t / k) tiles of 32 local rows (t = the request's tiles,
 *           counted from the tile of the first row its first query sees), part
 *           c holding tiles c*ceil(t/k) .. ; each part is written unmerged,
 *           normalised over its own rows: o [k][B][q_len][H][v_dim],
 *           lse [k][B][q_len][H] (an empty part: o = 0, lse = -inf; the sink,
 *           if any, joins part 0).  No workspace.  dcp_lse_merge over the
 *           N*k parts of all ranks gives the merged result directly. */

/* Packed records (page "MLA 的 DCP", section 5: the partial payload is
 * (512 + 4) x 2 bytes per (row, head), the output in bf16 and the LSE; page
 * "DCP", "merge: All-to-All": each rank sends head slice d to the rank that
 * owns it):
 * out_records  0: o and lse as above (float32).  1: `o` points to 16-bit
 *           records in head-owner order [N][k][B][q_len][H / N][v_dim + 4]
 *           (N = layout.n_stripes, k = num_splits with partials = 1, else 1;
 *           n_heads must be a multiple of N): per (row, head) the v_dim output
 *           values in bf16 (rounded to nearest even from the float32 result),
 *           then the float32 lse (lse_base) in the next two slots, low half
 *           first, then two zero slots -- the record of dcp_pack_heads, 8-byte
 *           aligned.  Block d is the piece of the all-to-all send buffer for
 *           owner d; the owner's dcp_merge_heads over the N (or N * k) blocks
 *           it receives gives the merged result.  `lse` is not used (may be
 *           NULL).  The float32 result is rounded once: the records equal
 *           dcp_pack_heads of the float32 outputs. */

/* Outputs in bf16 (page "MLA 的 DCP", section 5: the partial a rank hands to
 * the merge is (512 + 4) x 2 bytes per (row, head) -- the output in bf16
 * beside its LSE):
 * o_bf16  0: o is float32 as above.  1: `o` points to bf16 values in the same
 *         layout ([B][q_len][H][v_dim], or [k][B][q_len][H][v_dim] with
 *         partials = 1), each the float32 result rounded once to nearest
 *         even; lse stays float32.  dcp_lse_merge_bf16 merges such parts.
 *         With out_records = 1: DCP_EINVAL. */

/* Workspace bytes dcp_stripe_attn needs for `args` (pointers are not read). */
int dcp_stripe_attn_workspace(const dcp_attn_args* args, size_t* bytes);

/* dcp_stripe_attn -- one rank's local attention over its stripe, returning
 * (o_r, lse_r) (page "DCP", idea two; page "MLA 的 DCP", section 3). */
int dcp_stripe_attn(const dcp_attn_args* args, void* stream);

/* dcp_sparse_plan -- one rank's share of a global sparse selection.
 * Page "DCP", conditions for merging: sparse attention such as DSA's top-k
 * stays mergeable when the top-k is chosen globally and each rank attends only
 * to the selected tokens it owns.
 * topk_pos [batch][q_len][topk] int32 device: global positions chosen for each
 *          query token (shared by its heads); -1 marks an unused slot; the
 *          valid positions of one token must be distinct.  A position past
 *          the token's own (S - q_len + t) is ignored.
 * seq_len  [batch] int32 device, global lengths.
 * rows, bits [batch][stride] device out (stride >= q_len * topk): the kept
 *          entries of request b in (t, slot) order -- the rank's local row of
 *          the position and 1 << t; count [batch] int32 out: entries kept.
 * q_len > 32: DCP_EUNSUPPORTED. */
int dcp_sparse_plan(dcp_layout layout, int32_t rank, int32_t batch, int32_t q_len, int32_t topk,
                    const int32_t* topk_pos, const int32_t* seq_len, int32_t* rows, uint32_t* bits,
                    int32_t* count, int32_t stride, void* stream);

/* Head-return exchange (page "DCP", "merge: All-to-All"; page "MLA 的 DCP",
 * section 4, step 6): every rank packs its (o_r, lse_r) by destination -- the
 * rank that owns the heads -- into one buffer; after the all-to-all each
 * owner merges the N partials of its H/N heads.  Record of one (row, head):
 * v_dim bf16 output values (rounded to nearest even), the float32 lse in the
 * next two 16-bit slots, two zero slots: v_dim + 4 slots, 8-byte aligned.
 *
 * dcp_pack_heads -- o_r [rows][H][v_dim] fp32, lse_r [rows][H] fp32 (device;
 *   rows = B * q_len) -> send [N][rows][H/N][v_dim + 4] 16-bit slots (device):
 *   block d is what goes to rank d (heads d*H/N .. (d+1)*H/N - 1).
 *   H % N != 0 or v_dim % 4 != 0: DCP_EINVAL.
 * dcp_merge_heads -- recv [N][rows][v_dim + 4] (device; block r came from rank
 *   r, rows = B * q_len * H/N records) -> o [rows][v_dim] fp32, lse [rows] fp32
 *   (nullable), the exact merge in lse_base (that of the packed lse).  Parts
 *   with lse = -inf have zero weight and do not enter the result. */
int dcp_pack_heads(int32_t n_stripes, int64_t rows, int32_t n_heads, int32_t v_dim,
                   const float* o_r, const float* lse_r, void* send, void* stream);
int dcp_merge_heads(int32_t n_stripes, int64_t rows, int32_t v_dim, const void* recv,
                    int32_t lse_base, float* o, float* lse, void* stream);

/* dcp_stripe_attn_multi -- the stripe attentions of n ranks in one launch.
 * Page "DCP", idea two: every rank's local attention is independent of the
 * others', so the n calls args[0..n) can run as one launch that balances the
 * chunks of all ranks' requests over the GPU (on one GPU: the N-fold
 * parallelism of all stripes at once).  Each args[i] is a complete
 * dcp_stripe_attn argument block for its rank (own pool, block_table, o, lse,
 * sinks, sparse selection); everything else -- layout, shapes, q, seq_len,
 * scale, base, num_splits, window, softcap, bias_slopes, partials,
 * out_records, o_bf16 and whether a selection is given -- must be the same in all n
 * (else DCP_EINVAL).  The
 * workspace of args[0] serves the launch; size it with
 * dcp_stripe_attn_multi_workspace.  Results equal n dcp_stripe_attn calls.
 * 1 <= n <= 16 (n > 16: DCP_EUNSUPPORTED). */
int dcp_stripe_attn_multi_workspace(const dcp_attn_args* args, int32_t n, size_t* bytes);
int dcp_stripe_attn_multi(const dcp_attn_args* args, int32_t n, void* stream);

/* dcp_stripe_attn_noalloc -- dcp_stripe_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, semantics and results
 * as dcp_stripe_attn (bit for bit), except that args->workspace and
 * args->workspace_bytes are ignored: the chunk partials and chunk table go to
 * a fixed scratch buffer the library holds in device memory, one per GPU,
 * of dcp_stripe_attn_noalloc_max_bytes() bytes (64 MiB) -- every GPU the
 * library's kernels are loaded on holds it until the process ends.  A shape
 * whose workspace (dcp_stripe_attn_workspace) exceeds that size returns
 * DCP_ESCRATCH before any HIP call.  The call allocates and frees nothing;
 * the buffer needs no clearing (every byte a call reads was written by that
 * call's kernels).  All calls on one GPU share its buffer: calls that overlap
 * in time on one GPU (other streams, other threads) race and must not be
 * made; calls ordered on one stream are safe. */
int dcp_stripe_attn_noalloc(const dcp_attn_args* args, void* stream);
size_t dcp_stripe_attn_noalloc_max_bytes(void);

/* dcp_lse_merge -- exact merge of N stripes' partial results.
 * Page "DCP", "merge operator and numerical stability"; SGLang DCP docs,
 * "MLA decode dataflow": m = max_r lse_r, w_r = base^(lse_r - m),
 * o = sum_r w_r o_r / sum_r w_r, lse = m + log_base(sum_r w_r).
 * o_parts [N][rows][v_dim] fp32, lse_parts [N][rows] fp32 device, lse in
 * base e (lse_base 0) or 2 (lse_base 1).  Stripes with lse = -inf carry zero
 * weight and their o values are never used.  If every stripe of a row is
 * empty: o = 0, lse = -inf.  o [rows][v_dim], lse [rows] fp32 device out
 * (lse may be NULL).  v_dim % 4 == 0. */
int dcp_lse_merge(int32_t n_stripes, int64_t rows, int32_t v_dim,
                  const float* o_parts, const float* lse_parts, int32_t lse_base,
                  float* o, float* lse, void* stream);

/* dcp_lse_merge_bf16 -- the same exact merge over parts whose o is bf16 (the
 * o_bf16 outputs of dcp_stripe_attn; page "MLA 的 DCP", section 5, bf16
 * partials).  o_parts [N][rows][v_dim] bf16 (raw 16-bit values), lse_parts
 * [N][rows] fp32 device; the bf16 values are widened exactly and every sum
 * is float32.  o [rows][v_dim], lse [rows] fp32 device out (lse may be
 * NULL).  v_dim % 8 == 0 (16-byte loads).  Zero-weight parts as in
 * dcp_lse_merge. */
int dcp_lse_merge_bf16(int32_t n_parts, int64_t rows, int32_t v_dim,
                       const void* o_parts, const float* lse_parts, int32_t lse_base,
                       float* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCP_H */
