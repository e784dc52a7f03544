/*
 * A plain C client of libdcp: one decode step through the C ABI alone (no
 * Python, no torch), as a serving engine written in C or C++ would call it.
 *
 *   abi_client <input file> <output file>
 *
 * Input (little-endian): int32 B, H, N, I, P, q_len, lse_base; float scale;
 * int32 seq_len[B]; bf16 q[B][q_len][H][576]; bf16 kv rows of request 0, then
 * request 1, ... ([seq_len[b]][576] each, global positions 0 .. S_b - 1).
 * Output: float o[B][q_len][H][512], then float lse[B][q_len][H].
 *
 * The step: every rank's local lengths (dcp_local_count), every rank's paged
 * pool filled from all rows by the owner-filtered write (dcp_kv_write; each
 * rank keeps only the positions it owns), every rank's stripe attention
 * (dcp_stripe_attn with its own workspace), then the exact merge
 * (dcp_lse_merge).  Exit status 0 on success; any error is printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dcp.h"

#define D 576
#define DV 512

static int fail(const char* what, int code) {
  fprintf(stderr, "abi_client: %s: %s\n", what, code < 0 ? dcp_strerror(code) : "HIP error");
  return 1;
}

#define HIP(call)                                                               \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "abi_client: %s: %s\n", #call, hipGetErrorString(e_));    \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

#define DCP(call)                                  \
  do {                                             \
    int rc_ = (call);                              \
    if (rc_ != DCP_OK) return fail(#call, rc_);    \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n ? 0 : -1; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: abi_client <input> <output>\n");
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return fail("open input", 1);
  int32_t hdr[7];
  float scale;
  if (read_all(in, hdr, sizeof hdr) || read_all(in, &scale, sizeof scale)) return fail("read header", 1);
  const int32_t B = hdr[0], H = hdr[1], N = hdr[2], I = hdr[3], P = hdr[4], q_len = hdr[5], base = hdr[6];
  if (B < 1 || H < 1 || N < 1 || I < 1 || P < 1 || q_len < 1 || (base != 0 && base != 1)) return fail("header", 1);
  int32_t* seq = (int32_t*)malloc(sizeof(int32_t) * B);
  if (read_all(in, seq, sizeof(int32_t) * B)) return fail("read seq_len", 1);
  int64_t T = 0;
  for (int b = 0; b < B; ++b) {
    if (seq[b] < q_len) return fail("seq_len < q_len", 1);
    T += seq[b];
  }
  const int64_t rows = (int64_t)B * q_len * H;
  const size_t q_bytes = (size_t)rows * D * 2, kv_bytes = (size_t)T * D * 2;
  void* q_h = malloc(q_bytes);
  void* kv_h = malloc(kv_bytes);
  if (read_all(in, q_h, q_bytes) || read_all(in, kv_h, kv_bytes)) return fail("read q / kv", 1);
  fclose(in);

  const dcp_layout lay = {N, I, P};
  hipStream_t s;
  HIP(hipStreamCreate(&s));

  /* positions and request ids of all rows, and the lengths */
  int64_t* pos_h = (int64_t*)malloc(sizeof(int64_t) * T);
  int32_t* req_h = (int32_t*)malloc(sizeof(int32_t) * T);
  int64_t* len_h = (int64_t*)malloc(sizeof(int64_t) * B);
  for (int64_t b = 0, t = 0; b < B; ++b) {
    len_h[b] = seq[b];
    for (int32_t p = 0; p < seq[b]; ++p, ++t) {
      pos_h[t] = p;
      req_h[t] = (int32_t)b;
    }
  }
  void *q_d, *kv_d;
  int64_t *pos_d, *len_d, *count_d;
  int32_t *req_d, *seq_d, *status_d;
  HIP(hipMalloc(&q_d, q_bytes));
  HIP(hipMalloc(&kv_d, kv_bytes));
  HIP(hipMalloc((void**)&pos_d, sizeof(int64_t) * T));
  HIP(hipMalloc((void**)&req_d, sizeof(int32_t) * T));
  HIP(hipMalloc((void**)&len_d, sizeof(int64_t) * B));
  HIP(hipMalloc((void**)&count_d, sizeof(int64_t) * B * N));
  HIP(hipMalloc((void**)&seq_d, sizeof(int32_t) * B));
  HIP(hipMalloc((void**)&status_d, sizeof(int32_t)));
  HIP(hipMemcpy(q_d, q_h, q_bytes, hipMemcpyHostToDevice));
  HIP(hipMemcpy(kv_d, kv_h, kv_bytes, hipMemcpyHostToDevice));
  HIP(hipMemcpy(pos_d, pos_h, sizeof(int64_t) * T, hipMemcpyHostToDevice));
  HIP(hipMemcpy(req_d, req_h, sizeof(int32_t) * T, hipMemcpyHostToDevice));
  HIP(hipMemcpy(len_d, len_h, sizeof(int64_t) * B, hipMemcpyHostToDevice));
  HIP(hipMemcpy(seq_d, seq, sizeof(int32_t) * B, hipMemcpyHostToDevice));
  HIP(hipMemset(status_d, 0, sizeof(int32_t)));

  /* every rank's local length of every request */
  DCP(dcp_local_count(lay, NULL, len_d, B, count_d, s));
  int64_t* count_h = (int64_t*)malloc(sizeof(int64_t) * B * N);
  HIP(hipMemcpyAsync(count_h, count_d, sizeof(int64_t) * B * N, hipMemcpyDeviceToHost, s));
  HIP(hipStreamSynchronize(s));

  float *o_parts, *lse_parts, *o_d, *lse_d;
  HIP(hipMalloc((void**)&o_parts, sizeof(float) * N * rows * DV));
  HIP(hipMalloc((void**)&lse_parts, sizeof(float) * N * rows));
  HIP(hipMalloc((void**)&o_d, sizeof(float) * rows * DV));
  HIP(hipMalloc((void**)&lse_d, sizeof(float) * rows));

  for (int32_t r = 0; r < N; ++r) {
    /* this rank's page table: request b takes the next ceil(count / P) pages */
    int32_t cols = 1;
    for (int b = 0; b < B; ++b) {
      const int64_t pages = (count_h[(int64_t)b * N + r] + P - 1) / P;
      if (pages > cols) cols = (int32_t)pages;
    }
    int32_t* bt_h = (int32_t*)malloc(sizeof(int32_t) * B * cols);
    int64_t next = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t pages = (count_h[(int64_t)b * N + r] + P - 1) / P;
      for (int32_t c = 0; c < cols; ++c) bt_h[(int64_t)b * cols + c] = c < pages ? (int32_t)next++ : -1;
    }
    const int64_t num_pages = next > 0 ? next : 1;
    int32_t* bt_d;
    void* pool;
    HIP(hipMalloc((void**)&bt_d, sizeof(int32_t) * B * cols));
    HIP(hipMalloc(&pool, (size_t)num_pages * P * D * 2));
    HIP(hipMemcpy(bt_d, bt_h, sizeof(int32_t) * B * cols, hipMemcpyHostToDevice));
    HIP(hipMemsetAsync(pool, 0, (size_t)num_pages * P * D * 2, s));

    /* owner-filtered write of every row: the rank keeps the positions it owns */
    DCP(dcp_kv_write(lay, r, kv_d, D, T, pos_d, req_d, bt_d, B, cols, pool, num_pages, status_d, s));

    dcp_attn_args a;
    memset(&a, 0, sizeof a);
    a.layout = lay;
    a.rank = r;
    a.batch = B;
    a.q_len = q_len;
    a.n_heads = H;
    a.head_dim = D;
    a.v_dim = DV;
    a.q = q_d;
    a.pool = pool;
    a.num_pages = num_pages;
    a.block_table = bt_d;
    a.bt_cols = cols;
    a.seq_len = seq_d;
    a.scale = scale;
    a.lse_base = base;
    a.o = o_parts + (int64_t)r * rows * DV;
    a.lse = lse_parts + (int64_t)r * rows;
    a.status = status_d;
    size_t ws_bytes = 0;
    DCP(dcp_stripe_attn_workspace(&a, &ws_bytes));
    void* ws = NULL;
    if (ws_bytes > 0) HIP(hipMalloc(&ws, ws_bytes));
    a.workspace = ws;
    a.workspace_bytes = ws_bytes;
    DCP(dcp_stripe_attn(&a, s));
    HIP(hipStreamSynchronize(s));   /* before this rank's buffers are freed */
    HIP(hipFree(ws));
    HIP(hipFree(pool));
    HIP(hipFree(bt_d));
    free(bt_h);
  }
  DCP(dcp_lse_merge(N, rows, DV, o_parts, lse_parts, base, o_d, lse_d, s));

  float* o_h = (float*)malloc(sizeof(float) * rows * DV);
  float* lse_h = (float*)malloc(sizeof(float) * rows);
  int32_t status_h = 0;
  HIP(hipMemcpyAsync(o_h, o_d, sizeof(float) * rows * DV, hipMemcpyDeviceToHost, s));
  HIP(hipMemcpyAsync(lse_h, lse_d, sizeof(float) * rows, hipMemcpyDeviceToHost, s));
  HIP(hipMemcpyAsync(&status_h, status_d, sizeof(int32_t), hipMemcpyDeviceToHost, s));
  HIP(hipStreamSynchronize(s));
  if (status_h != DCP_OK) return fail("device status", status_h);

  FILE* out = fopen(argv[2], "wb");
  if (!out) return fail("open output", 1);
  if (fwrite(o_h, sizeof(float), rows * DV, out) != (size_t)(rows * DV) ||
      fwrite(lse_h, sizeof(float), rows, out) != (size_t)rows)
    return fail("write output", 1);
  fclose(out);
  printf("abi_client: ok (B=%d H=%d N=%d I=%d P=%d q_len=%d, %lld rows written)\n", B, H, N, I, P, q_len,
         (long long)T);
  return 0;
}
