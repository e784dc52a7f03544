/* Host-side argument checking of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (no GPU needed).
 *
 * Every call below is rejected, or answered, on the host before any kernel
 * is enqueued: bad layouts and ranks, NULL buffers with non-zero sizes,
 * negative and huge sizes, unsupported shapes, workspace-size queries over a
 * grid of shapes up to the int32 limits of the argument block (so the plan's
 * size arithmetic runs on extreme values), and the allocation-free entry
 * point's scratch limit.  A sanitizer report aborts the process; on success
 * it prints the number of checks and exits 0. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dcp.h"

static int checks = 0, failures = 0;

#define CHECK(expr, want)                                                                      \
  do {                                                                                         \
    const int got_ = (expr);                                                                   \
    ++checks;                                                                                  \
    if (got_ != (want)) {                                                                      \
      ++failures;                                                                              \
      fprintf(stderr, "%s:%d: %s returned %d (%s), want %d\n", __FILE__, __LINE__, #expr, got_, \
              dcp_strerror(got_), (want));                                                     \
    }                                                                                          \
  } while (0)

static void* const FAKE = (void*)0x1000;   /* never dereferenced: every call fails validation first */

static dcp_attn_args base_args(void) {
  dcp_attn_args a;
  memset(&a, 0, sizeof a);
  a.layout.n_stripes = 8;
  a.layout.interleave = 1;
  a.layout.page_size = 64;
  a.rank = 0;
  a.batch = 2;
  a.q_len = 1;
  a.n_heads = 16;
  a.head_dim = 576;
  a.v_dim = 512;
  a.q = FAKE;
  a.pool = FAKE;
  a.num_pages = 4;
  a.block_table = FAKE;
  a.bt_cols = 4;
  a.seq_len = FAKE;
  a.scale = 0.07f;
  a.num_splits = 2;
  a.o = FAKE;
  a.lse = FAKE;
  return a;
}

static void strerror_and_version(void) {
  for (int c = -10; c <= 10; ++c) {
    ++checks;
    if (dcp_strerror(c) == NULL || dcp_strerror(c)[0] == 0) {
      ++failures;
      fprintf(stderr, "dcp_strerror(%d) is empty\n", c);
    }
  }
  ++checks;
  if (dcp_abi_version() < 1) {
    ++failures;
    fprintf(stderr, "dcp_abi_version() < 1\n");
  }
}

static void layouts(void) {
  const dcp_layout bad[] = {{0, 1, 64}, {8, 0, 64}, {8, 1, 0}, {8, 3, 64}, {-2, 1, 64}, {8, 64, 48},
                            {8, INT32_MAX, 64}, {8, 1, INT32_MIN}};
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    const dcp_layout l = bad[i];
    CHECK(dcp_slot_map(l, 0, FAKE, NULL, 4, NULL, 0, 0, FAKE, FAKE, FAKE, NULL, NULL), DCP_EINVAL);
    CHECK(dcp_local_count(l, NULL, FAKE, 4, FAKE, NULL), DCP_EINVAL);
    dcp_attn_args a = base_args();
    a.layout = l;
    CHECK(dcp_stripe_attn(&a, NULL), DCP_EINVAL);
  }
}

static void layout_kernels(void) {
  const dcp_layout l = {8, 1, 64};
  CHECK(dcp_slot_map(l, 8, FAKE, NULL, 4, NULL, 0, 0, FAKE, FAKE, FAKE, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_slot_map(l, 0, NULL, NULL, 4, NULL, 0, 0, FAKE, FAKE, FAKE, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_slot_map(l, 0, FAKE, NULL, -1, NULL, 0, 0, FAKE, FAKE, FAKE, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_slot_map(l, 0, FAKE, NULL, INT64_MIN, NULL, 0, 0, FAKE, FAKE, FAKE, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_slot_map(l, 0, NULL, NULL, 0, NULL, 0, 0, NULL, NULL, NULL, NULL, NULL), DCP_OK);
  CHECK(dcp_local_count(l, NULL, NULL, 3, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_local_count(l, NULL, FAKE, -3, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_local_count(l, NULL, NULL, 0, NULL, NULL), DCP_OK);
  CHECK(dcp_kv_write(l, 0, FAKE, 577, 4, FAKE, NULL, FAKE, 1, 1, FAKE, 1, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_kv_write(l, 0, NULL, 576, 4, FAKE, NULL, FAKE, 1, 1, FAKE, 1, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_kv_write(l, 0, FAKE, 576, -4, FAKE, NULL, FAKE, 1, 1, FAKE, 1, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_kv_write(l, 0, FAKE, 576, 4, FAKE, NULL, NULL, 1, 1, FAKE, 1, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_kv_write(l, 0, FAKE, 576, 4, FAKE, NULL, FAKE, 1, 1, FAKE, 0, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_kv_write(l, 0, NULL, 576, 0, NULL, NULL, FAKE, 1, 1, FAKE, 1, NULL, NULL), DCP_OK);
  CHECK(dcp_relayout(l, 0, 576, FAKE, 1, 64, FAKE, 1, FAKE, FAKE, 65536, 100, FAKE, 1, FAKE, 1, NULL, NULL),
        DCP_EUNSUPPORTED);
  CHECK(dcp_relayout(l, 0, 577, FAKE, 1, 64, FAKE, 1, FAKE, FAKE, 2, 100, FAKE, 1, FAKE, 1, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_relayout(l, 9, 576, FAKE, 1, 64, FAKE, 1, FAKE, FAKE, 2, 100, FAKE, 1, FAKE, 1, NULL, NULL), DCP_EINVAL);
  CHECK(dcp_sparse_plan(l, 0, 2, 33, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 33 * 8, NULL), DCP_EUNSUPPORTED);
  CHECK(dcp_sparse_plan(l, 0, 2, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 15, NULL), DCP_EINVAL);
  CHECK(dcp_sparse_plan(l, 0, 2, 2, 8, NULL, FAKE, FAKE, FAKE, FAKE, 16, NULL), DCP_EINVAL);
}

static void merges(void) {
  CHECK(dcp_lse_merge(0, 4, 512, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge(8, -1, 512, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge(8, 4, 510, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge(8, 4, 512, FAKE, FAKE, 2, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge(8, 4, 512, NULL, FAKE, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge(8, 0, 512, NULL, NULL, 0, NULL, NULL, NULL), DCP_OK);
  CHECK(dcp_lse_merge(8, INT64_MAX, 512, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EUNSUPPORTED);
  CHECK(dcp_lse_merge_bf16(0, 4, 512, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge_bf16(8, -1, 512, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge_bf16(8, 4, 508, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge_bf16(8, 4, 512, FAKE, FAKE, 2, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge_bf16(8, 4, 512, FAKE, NULL, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge_bf16(8, 4, 512, FAKE, FAKE, 0, NULL, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_lse_merge_bf16(8, 0, 512, NULL, NULL, 0, NULL, NULL, NULL), DCP_OK);
  CHECK(dcp_lse_merge_bf16(8, INT64_MAX, 512, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EUNSUPPORTED);
  CHECK(dcp_lse_merge_bf16(INT32_MAX, INT64_MAX / 8, 512, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EUNSUPPORTED);
  CHECK(dcp_lse_merge_bf16(INT32_MAX, ((int64_t)1 << 33) - 4, 512, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EUNSUPPORTED);
  CHECK(dcp_lse_merge_bf16(2, 4, INT32_MAX - 3, FAKE, FAKE, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_pack_heads(8, 4, 12, 512, FAKE, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_pack_heads(8, 4, 16, 510, FAKE, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_pack_heads(8, 4, 16, 512, NULL, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_pack_heads(8, 0, 16, 512, NULL, NULL, NULL, NULL), DCP_OK);
  CHECK(dcp_pack_heads(8, INT64_MAX, 16, 512, FAKE, FAKE, FAKE, NULL), DCP_EUNSUPPORTED);
  CHECK(dcp_pack_heads(8, INT64_MAX / 2048, INT32_MAX - 7, 512, FAKE, FAKE, FAKE, NULL), DCP_EUNSUPPORTED);
  CHECK(dcp_merge_heads(0, 4, 512, FAKE, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_merge_heads(8, 4, 512, FAKE, 3, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_merge_heads(8, 4, 512, NULL, 0, FAKE, FAKE, NULL), DCP_EINVAL);
  CHECK(dcp_merge_heads(8, INT64_MAX, 512, FAKE, 0, FAKE, FAKE, NULL), DCP_EUNSUPPORTED);
}

static void stripe_attn_arguments(void) {
  dcp_attn_args a;
#define BAD(field, value, want)          \
  a = base_args();                       \
  a.field = (value);                     \
  CHECK(dcp_stripe_attn(&a, NULL), want);
  BAD(rank, 8, DCP_EINVAL);
  BAD(rank, -1, DCP_EINVAL);
  BAD(batch, 0, DCP_EINVAL);
  BAD(batch, INT32_MIN, DCP_EINVAL);
  BAD(q_len, 0, DCP_EINVAL);
  BAD(n_heads, -5, DCP_EINVAL);
  BAD(head_dim, 512, DCP_EUNSUPPORTED);
  BAD(v_dim, 576, DCP_EUNSUPPORTED);
  BAD(num_pages, 0, DCP_EINVAL);
  BAD(bt_cols, 0, DCP_EINVAL);
  BAD(lse_base, 2, DCP_EINVAL);
  BAD(num_splits, -1, DCP_EINVAL);
  BAD(q, NULL, DCP_EINVAL);
  BAD(pool, NULL, DCP_EINVAL);
  BAD(seq_len, NULL, DCP_EINVAL);
  BAD(o, NULL, DCP_EINVAL);
  BAD(lse, NULL, DCP_EINVAL);
  BAD(window, -1, DCP_EINVAL);
  BAD(softcap, -1.0f, DCP_EINVAL);
  BAD(partials, 2, DCP_EINVAL);
  BAD(out_records, 2, DCP_EINVAL);
  BAD(o_bf16, 2, DCP_EINVAL);
  BAD(o_bf16, -1, DCP_EINVAL);
#undef BAD
  /* bf16 outputs and records are two output forms: not both */
  a = base_args();
  a.out_records = 1;
  a.o_bf16 = 1;
  CHECK(dcp_stripe_attn(&a, NULL), DCP_EINVAL);
  /* splits need a workspace: rejected before launch when none (or too small) is given */
  a = base_args();
  a.num_splits = 3;
  CHECK(dcp_stripe_attn(&a, NULL), DCP_EINVAL);
  size_t need = 0;
  CHECK(dcp_stripe_attn_workspace(&a, &need), DCP_OK);
  a.workspace = FAKE;
  a.workspace_bytes = need - 1;
  CHECK(dcp_stripe_attn(&a, NULL), DCP_EINVAL);
  CHECK(dcp_stripe_attn_workspace(&a, NULL), DCP_EINVAL);
  CHECK(dcp_stripe_attn_workspace(NULL, &need), DCP_EINVAL);
  /* records need whole head slices per stripe */
  a = base_args();
  a.out_records = 1;
  a.n_heads = 12;
  CHECK(dcp_stripe_attn(&a, NULL), DCP_EINVAL);
  /* the allocation-free entry point: a shape past its fixed scratch */
  a = base_args();
  a.batch = 4096;
  a.bt_cols = 4096;
  a.num_splits = 64;
  CHECK(dcp_stripe_attn_workspace(&a, &need), DCP_OK);
  ++checks;
  if (need <= dcp_stripe_attn_noalloc_max_bytes()) ++failures;
  CHECK(dcp_stripe_attn_noalloc(&a, NULL), DCP_ESCRATCH);
  /* several ranks */
  dcp_attn_args arr[17];
  for (int i = 0; i < 17; ++i) {
    arr[i] = base_args();
    arr[i].rank = i % 8;
  }
  CHECK(dcp_stripe_attn_multi(arr, 17, NULL), DCP_EUNSUPPORTED);
  CHECK(dcp_stripe_attn_multi(arr, 0, NULL), DCP_EINVAL);
  CHECK(dcp_stripe_attn_multi(NULL, 2, NULL), DCP_EINVAL);
  arr[1].batch = 3;
  CHECK(dcp_stripe_attn_multi(arr, 2, NULL), DCP_EINVAL);
  /* every rank of one launch writes the same output form */
  arr[1] = base_args();
  arr[1].rank = 1;
  arr[1].o_bf16 = 1;
  CHECK(dcp_stripe_attn_multi(arr, 2, NULL), DCP_EINVAL);
}

/* Workspace queries over a grid of shapes, extreme values included: the plan's
 * arithmetic must stay defined (the sanitizer aborts on signed overflow) and
 * answer OK or DCP_EUNSUPPORTED. */
static void workspace_grid(void) {
  const int32_t batches[] = {1, 2, 64, 4096, 65535, INT32_MAX};
  const int32_t qlens[] = {1, 4, 32, 4096, INT32_MAX};
  const int32_t heads[] = {1, 16, 96, 128, 384, INT32_MAX};
  const int32_t splits[] = {0, 1, 4, 1000, INT32_MAX};
  const int32_t cols[] = {1, 256, 65536, INT32_MAX};
  const int32_t pages[] = {8, 64, 4096, 1 << 30};
  for (size_t ib = 0; ib < sizeof batches / sizeof batches[0]; ++ib)
    for (size_t iq = 0; iq < sizeof qlens / sizeof qlens[0]; ++iq)
      for (size_t ih = 0; ih < sizeof heads / sizeof heads[0]; ++ih)
        for (size_t is = 0; is < sizeof splits / sizeof splits[0]; ++is)
          for (size_t ic = 0; ic < sizeof cols / sizeof cols[0]; ++ic)
            for (size_t ip = 0; ip < sizeof pages / sizeof pages[0]; ++ip)
              for (int partials = 0; partials < 2; ++partials) {
                dcp_attn_args a = base_args();
                a.batch = batches[ib];
                a.q_len = qlens[iq];
                a.n_heads = heads[ih];
                a.num_splits = splits[is];
                a.bt_cols = cols[ic];
                a.layout.page_size = pages[ip];
                a.partials = partials && splits[is] > 0;
                size_t need = 0;
                const int rc = dcp_stripe_attn_workspace(&a, &need);
                ++checks;
                if (rc != DCP_OK && rc != DCP_EUNSUPPORTED && rc != DCP_EINVAL) {
                  ++failures;
                  fprintf(stderr, "workspace(B=%d q_len=%d H=%d splits=%d cols=%d P=%d partials=%d) = %d\n",
                          a.batch, a.q_len, a.n_heads, a.num_splits, a.bt_cols, a.layout.page_size, a.partials, rc);
                }
                dcp_attn_args two[2] = {a, a};
                two[1].rank = 1;
                const int rm = dcp_stripe_attn_multi_workspace(two, 2, &need);
                ++checks;
                if (rm != DCP_OK && rm != DCP_EUNSUPPORTED && rm != DCP_EINVAL) ++failures;
              }
}

int main(void) {
  strerror_and_version();
  layouts();
  layout_kernels();
  merges();
  stripe_attn_arguments();
  workspace_grid();
  if (failures) {
    fprintf(stderr, "abi_errors: %d of %d checks failed\n", failures, checks);
    return 1;
  }
  printf("abi_errors: %d checks ok\n", checks);
  return 0;
}
