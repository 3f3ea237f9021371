// Paged decode path: host entry points implemented in idx_decode.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "idx_topk.h"

namespace idxk {

size_t decode_workspace_bytes(int32_t B, int32_t max_pages, int32_t page_size, int32_t K);

int decode_paged(const uint8_t* q, const float* q_scale, const uint8_t* k_cache, const float* k_scale,
                 const float* w, const int32_t* page_table, const int32_t* seq_lens, int32_t B,
                 int32_t max_pages, int32_t page_size, int32_t num_pages, int32_t K, int32_t* out_idx,
                 void* workspace, size_t workspace_bytes, hipStream_t stream, const idx_topk_opts* opts,
                 float* scores_out = nullptr);

// The allocation-free variant: the same call with a static per-GPU scratch.
int decode_paged_noalloc(const uint8_t* q, const float* q_scale, const uint8_t* k_cache, const float* k_scale,
                         const float* w, const int32_t* page_table, const int32_t* seq_lens, int32_t B,
                         int32_t max_pages, int32_t page_size, int32_t num_pages, int32_t K, int32_t* out_idx,
                         hipStream_t stream);

}  // namespace idxk
