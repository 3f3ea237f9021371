// BF16 stream scan and the streaming-floor kernel: host entry points
// implemented in idx_scan.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "idx_topk.h"

namespace idxk {

size_t scan_bf16_workspace_bytes(int32_t B, int32_t N, int32_t K);

int scan_bf16(const uint16_t* q, const float* w, const uint16_t* k, const int32_t* lens, int32_t B, int32_t N,
              int32_t K, int32_t* out_idx, void* workspace, size_t workspace_bytes, hipStream_t stream,
              const idx_topk_opts* opts);

const float* scan_bf16_scores(const void* workspace, int32_t B, int32_t N);

int stream_floor(const void* src, int64_t n_records, float* dst, hipStream_t stream);

}  // namespace idxk
