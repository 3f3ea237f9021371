// Launch arguments of the dense-matrix top-K (idx_rows.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxk {

// Dense rows: row t's scores at scores + t*ld, position s at [s], range
// [row_start[t], row_end[t]).  Paged decode rows (table != null): row b
// covers logical positions [0, row_end[b]) (the sequence lengths, row_start
// unused), is invalid when one of the page ids it uses lies outside
// [0, num_pages), and emits physical slots table[b*max_pages + i/64]*64 + i%64.
struct RowsArgs {
  const float* scores;
  int64_t ld;
  const int32_t* row_start;
  const int32_t* row_end;
  int32_t Q, N, K;
  int32_t* out;    // [Q][K]
  uint32_t* ctrl;  // control words with the stats copies, or null
  const int32_t* table;
  int32_t max_pages;
  int32_t num_pages;
  // Optional pre-gathered lists (paged rows): workgroup g of k_rows_gather
  // (gsplit a power of two <= kMaxGatherSplit per row) stores the keys at or above the
  // row's sampled cut found in slice g of the row into its own region
  // (gcap entries) and their number into gcnt[t*gsplit + g].
  uint32_t* gkey;  // [Q][gsplit][gcap] order-preserving keys, or null
  int32_t* gid;    // [Q][gsplit][gcap] logical positions
  uint32_t* gcnt;  // [Q][gsplit]
  int32_t gcap, gsplit;
  // Optional candidates filtered by the paged decode's scoring kernel
  // (instead of the pre-gather): sequence t's workgroups are
  // g = dplan[t].x + i for i < dplan[t].y; wave v of workgroup g stored
  // dcnt[t * kDecodeCntStride + 4i + v] (order-preserving key, logical
  // position) pairs, the first dseg of them at dcand[(4g + v) * dseg]; they
  // are the keys of the sequence at or above one threshold.
  const uint2* dcand;
  const uint32_t* dcnt;
  const uint2* dplan;
  int32_t dseg;
};

constexpr int kMaxGatherSplit = 32;
// Count slots per decode sequence: four waves for each of at most 512
// scoring workgroups.
constexpr int kDecodeCntStride = 2048;

// Launch the pre-gather and the per-row select (paged rows when table is
// set, dense rows otherwise; gkey must be set).
int launch_topk_rows_gathered(const RowsArgs& A, hipStream_t stream);

// The per-sequence select of the paged decode over the candidates its
// scoring kernel filtered (dcnt, dcand, dplan set; no pre-gather).
int launch_topk_rows_filtered(const RowsArgs& A, hipStream_t stream);

// The per-row select alone, for dense rows (table must be null).
int launch_topk_rows(const RowsArgs& A, hipStream_t stream);

}  // namespace idxk
