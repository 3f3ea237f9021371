// Internal launch arguments, capacities and candidate sources.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "idx_common.hpp"
#include "idx_topk.h"

namespace idxk {

// Threshold sampler ("3.2 Sampled threshold": about 0.5% of the row, spread
// over it, aiming at about 2K candidates).
constexpr int kSampleStride = IDX_TOPK_SAMPLE_STRIDE;
constexpr int kSampleOffset = IDX_TOPK_SAMPLE_OFFSET;
constexpr int kSampleTarget = IDX_TOPK_SAMPLE_TARGET;
constexpr int kMaxSamples = 2048;  // longer rows widen the stride instead

// Candidate capacities per row.  Two rows per workgroup keep 2 x 4096
// candidates (64 KiB) on chip so that two workgroups fit one CU's 160 KiB of
// LDS; the spill area in the workspace doubles the capacity ("4.5 Overflow
// spill area").
constexpr int kBQ = 2;
constexpr int kLdsCap = 4096;
constexpr int kSpillCap = 4096;

// Control words at the start of every workspace.
constexpr int kCtrlWords = 16;
constexpr int kCtrlFail = 0;   // number of rows on the failure list
constexpr int kStatsOff = 8;   // idx_topk_stats, in declaration order
constexpr int kStRows = 0, kStFast = 1, kStUnder = 2, kStOver = 3, kStSpilled = 4,
              kStRepaired = 5, kStTrivial = 6, kStBad = 7;

__host__ __device__ inline int repair_grid(int rows) { return rows < 256 ? (rows > 0 ? rows : 1) : 256; }

struct PrefillArgs {
  const uint8_t* q;
  const float* q_scale;
  const uint8_t* k;
  const float* k_scale;
  const float* w;
  const int32_t* row_start;
  const int32_t* row_end;
  int32_t Q, N, K;
  float* tau;           // [Q]
  int32_t* out;         // [Q][K]
  uint32_t* spill_key;  // [Q][spill_cap]
  int32_t* spill_idx;   // [Q][spill_cap]
  int32_t lds_cap, spill_cap, cap_total;
  int32_t* fail_list;   // [Q]
  uint32_t* ctrl;       // kCtrlWords
  uint32_t* scratch;    // [repair_grid(Q)][N]
  float* dbg_scores;    // [Q][N] or null
  int32_t force_tau;
  float tau_value;
  hipEvent_t ev_main_start, ev_main_stop;  // host-side only: timing hooks
};

struct SampleGeom {
  int n, stride, r;
};

// Sample lattice of a row of length L: positions OFFSET + stride*i < L.  Rows
// that fit the candidate capacity need no threshold (n = 0: tau = -inf).
__device__ inline SampleGeom sample_geom(int L, int cap_total) {
  SampleGeom g{0, kSampleStride, 0};
  if (L <= cap_total || L <= kSampleOffset) return g;
  const int64_t span = (int64_t)L - kSampleOffset;
  int64_t stride = kSampleStride;
  if ((span + stride - 1) / stride > kMaxSamples) stride = (span + kMaxSamples - 1) / kMaxSamples;
  g.stride = (int)stride;
  g.n = (int)((span + stride - 1) / stride);
  const int64_t r = ((int64_t)g.n * kSampleTarget + L - 1) / L;
  g.r = (int)(r < 1 ? 1 : (r > g.n ? g.n : r));
  return g;
}

// ------------------------------------------------ candidate sources for select

struct SrcLds {
  const uint32_t* k;
  __device__ uint32_t key(int i) const { return k[i]; }
  __device__ int32_t id(int i) const { return i; }
};

struct SrcLdsSpill {
  const uint32_t* lk;
  const int32_t* li;
  int nl;
  const uint32_t* gk;
  const int32_t* gi;
  __device__ uint32_t key(int i) const { return i < nl ? lk[i] : gk[i - nl]; }
  __device__ int32_t id(int i) const { return i < nl ? li[i] : gi[i - nl]; }
};

// ------------------------------------------------ key addressing

// Logical key position -> row of the [*, 128] key array (and of the scale
// array, which is indexed the same way).
struct MapIdentity {
  __device__ int64_t operator()(int i) const { return i; }
};

// Paged cache with 64-token pages: position i of a sequence lives in page
// table[i / 64], slot i % 64 ("DSA TopK Indexer", contest report page).
struct MapPaged {
  const int32_t* table;
  __device__ int64_t operator()(int i) const { return (int64_t)table[i >> 6] * 64 + (i & 63); }
};

// Sample i of a row starting at s0 sits at position s0 + OFFSET + stride * i.
template <class M>
struct MapLattice {
  M inner;
  int s0, stride;
  __device__ int64_t operator()(int i) const { return inner(s0 + kSampleOffset + stride * i); }
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Scores of the 64 positions key0 .. key0+63 for BQ query rows; lane l gets
// position key0 + l.  Positions are clamped into [lo, hi-1] for the loads
// (callers mask by range), so every access stays inside the key arrays.
template <int BQ, class M>
__device__ __forceinline__ void score_tile(const QOp (&qo)[BQ], const uint8_t* k, const float* k_scale,
                                           const M& map, int key0, int lo, int hi, uint32_t lane,
                                           float (&sc)[BQ]) {
  v8i kb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = clampi(key0 + sub_off(c) + (int)(lane & 15), lo, hi - 1);
    kb[c] = ld32(k + map(i) * kD + 32 * (lane >> 4));
  }
  const float ks = k_scale[map(clampi(key0 + (int)lane, lo, hi - 1))];
#pragma unroll
  for (int r = 0; r < BQ; ++r) sc[r] = tile_sum(qo[r], kb) * ks;
}

// Threshold of one row from its sample lattice: score the samples exactly
// like the main pass (so the sampled keys reproduce bit-identical scores
// there) and return the r-th largest.  Whole workgroup calls.
template <class M>
__device__ float sample_tau(const QOp& qo, const uint8_t* k, const float* k_scale, const M& map, int s0,
                            const SampleGeom& sg, uint32_t* s_samp, SelShared& sh, int tid) {
  const uint32_t lane = tid & 63;
  const int wave = tid >> 6;
  const MapLattice<M> lm{map, s0, sg.stride};
  const QOp qa[1] = {qo};
  for (int tile = wave; tile * kTile < sg.n; tile += kWaves) {
    float sc[1];
    score_tile<1>(qa, k, k_scale, lm, tile * kTile, 0, sg.n, lane, sc);
    const int i = tile * kTile + (int)lane;
    if (i < sg.n) s_samp[i] = f2key(sc[0]);
  }
  __syncthreads();
  const SrcLds src{s_samp};
  const SelResult sel = radix_select(src, sg.n, sg.r, sh, tid, false, false);
  return key2f(sel.prefix);
}

// Candidate source over a repair scratch row: element i is position s0 + i.
template <class IdMap>
struct SrcScratchT {
  const uint32_t* k;
  int32_t s0;
  IdMap ids;
  __device__ uint32_t key(int i) const { return k[i]; }
  __device__ int32_t id(int i) const { return ids(s0 + i); }
};

struct IdIdentity {
  __device__ int32_t operator()(int i) const { return i; }
};
struct IdPaged {
  const int32_t* table;
  __device__ int32_t operator()(int i) const { return table[i >> 6] * 64 + (i & 63); }
};

// Exact selection for one row without a threshold: rescore positions
// [s0, s1) into scratch (order-preserving keys), build the top-byte
// histogram on the way, finish the radix select over scratch and emit
// ids(i) of the winners into out[0..K).  Whole workgroup calls.
template <class M, class IdMap>
__device__ void repair_row(const QOp& qo, const uint8_t* k, const float* k_scale, const M& map,
                           const IdMap& ids, int s0, int s1, int K, int32_t* out, uint32_t* scratch,
                           SelShared& sh, int tid) {
  const uint32_t lane = tid & 63;
  const int wave = tid >> 6;
  const int L = s1 - s0, kr = L < K ? L : K;
  for (int i = tid; i < 256; i += kWG) sh.hist[i] = 0u;
  __syncthreads();
  const QOp qa[1] = {qo};
  const int tile_lo = s0 >> 6, tile_hi = (s1 + 63) >> 6;
  for (int tile = tile_lo + wave; tile < tile_hi; tile += kWaves) {
    const int key0 = tile << 6;
    float sc[1];
    score_tile<1>(qa, k, k_scale, map, key0, s0, s1, lane, sc);
    const int my = key0 + (int)lane;
    const bool valid = my >= s0 && my < s1;
    const uint32_t key = f2key(sc[0]);
    if (valid) scratch[my - s0] = key;
    hist_add(sh.hist, key >> 24, valid);
  }
  __syncthreads();
  const SrcScratchT<IdMap> src{scratch, s0, ids};
  const SelResult sel = (L > kr) ? radix_select(src, L, kr, sh, tid, true, true) : SelResult{0u, 0u, kr};
  emit_selection(src, L, sel, kr, K, out, sh, tid);
}

int launch_prefill(const PrefillArgs& A, hipStream_t stream);

}  // namespace idxk
