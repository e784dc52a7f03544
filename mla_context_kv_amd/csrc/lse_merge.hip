// dcp_lse_merge: exact merge of N stripes' partial results (the kernel and
// its derivation are in merge_impl.h).
#include "merge_impl.h"

extern "C" int dcp_lse_merge(int32_t n_stripes, int64_t rows, int32_t v_dim, const float* o_parts,
                             const float* lse_parts, int32_t lse_base, float* o, float* lse,
                             void* stream) {
  if (n_stripes < 1 || rows < 0 || v_dim <= 0 || v_dim % 4 != 0) return DCP_EINVAL;
  if (lse_base != 0 && lse_base != 1) return DCP_EINVAL;
  if (rows > 0 && (o_parts == nullptr || lse_parts == nullptr || o == nullptr)) return DCP_EINVAL;
  if (rows == 0) return DCP_OK;
  return dcp::launch_lse_merge(n_stripes, rows, v_dim, o_parts, lse_parts, lse_base, lse_base, o,
                               lse, (hipStream_t)stream);
}
