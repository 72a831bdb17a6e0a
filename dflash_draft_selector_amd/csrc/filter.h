// Internal interface of the filtered-target verify (k_filter.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dflash2_internal.h"

namespace df2 {

struct FilterWs {
  unsigned long long* lists;      // [nrows][8 * nchunks][top_k] each sub-chunk's top_k, best first (0 = none)
  int* flags;                     // [nrows][8 * nchunks] 1: the sub-chunk holds +inf or NaN
};
FilterWs carve_filter(Carver& c, int64_t nrows, int64_t vocab);

hipError_t launch_spec_accept_filtered(const uint16_t* target, int64_t ld, int64_t batch_stride,
                                       const int32_t* tokens, const int32_t* cand_idx, const float* q, int batch,
                                       int K, int vocab, float temperature, int top_k, float top_p, uint64_t seed,
                                       int32_t* out_tokens, int32_t* n_accepted, int32_t* row_status, FilterWs ws,
                                       hipStream_t s);

}  // namespace df2
