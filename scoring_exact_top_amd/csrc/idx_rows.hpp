// Launch arguments of the dense-matrix top-K (idx_rows.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxk {

struct RowsArgs {
  const float* scores;  // row t's scores at scores + t*ld; position s at [s]
  int64_t ld;
  const int32_t* row_start;
  const int32_t* row_end;
  int32_t Q, N, K;
  int32_t* out;    // [Q][K]
  uint32_t* ctrl;  // control words with the stats copies, or null
};

int launch_topk_rows(const RowsArgs& A, hipStream_t stream);

}  // namespace idxk
