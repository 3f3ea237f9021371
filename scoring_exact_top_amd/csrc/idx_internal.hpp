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

// Main kernel geometry: 8 waves (two per SIMD), one query row per wave.
constexpr int kMainWaves = 8;
constexpr int kMainThreads = 64 * kMainWaves;
// Candidates per row: (key, id) pairs are staged in a 2048-entry LDS area per
// wave (8 x 16 KiB of the CU's 160 KiB) and flushed to the row's candidate
// list in the workspace whenever the stage is nearly full ("4.5 Overflow
// spill area": on-chip first, device memory beyond).  The certificate's
// capacity is the list length kCandCap.
constexpr int kStage = 2048;
constexpr int kLdsCap = 4096;    // default on-chip share of the capacity
constexpr int kSpillCap = 4096;  // default device-memory share
constexpr int kCandCap = kLdsCap + kSpillCap;
// Paired-row kernel: each (row, wave) owns a private segment of the row's
// candidate list ("4.3 Candidate layout: warp-private segments"): an LDS
// stage of kSegStage entries flushed in bulk to kSegCap entries of the
// workspace, so slot positions come from a scalar count with no atomics.
constexpr int kSegStage = 1024;
constexpr int kSegCap = kCandCap / 4;

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
  uint8_t* kt;          // [ntiles][8][64][16] keys relaid in MFMA lane order
  uint32_t* cand_key;   // [Q][kCandCap] flushed candidate keys
  int32_t* cand_idx;    // [Q][kCandCap] flushed candidate ids
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

// Candidates of the paired-row kernel: four wave segments of one row in the
// workspace, o[s] = first element of segment s, raw FP32 score bits.
struct SrcSeg4 {
  const uint32_t* gk;  // [4][kSegCap]
  const int32_t* gi;
  int o1, o2, o3;
  __device__ int at(int i) const {
    const int s = (i >= o1) + (i >= o2) + (i >= o3);
    const int base = s == 0 ? 0 : s == 1 ? o1 : s == 2 ? o2 : o3;
    return s * kSegCap + (i - base);
  }
  __device__ uint32_t key(int i) const { return f2key(__uint_as_float(gk[at(i)])); }
  __device__ int32_t id(int i) const { return gi[at(i)]; }
};

// Candidates of the paired-row kernel: [0, nl) in LDS, the rest in the
// row's spill area of the workspace.
struct SrcLdsSpill {
  const uint32_t* lk;
  const int32_t* li;
  int nl;
  const uint32_t* gk;
  const int32_t* gi;
  __device__ uint32_t key(int i) const { return i < nl ? lk[i] : gk[i - nl]; }
  __device__ int32_t id(int i) const { return i < nl ? li[i] : gi[i - nl]; }
};

// Main-kernel candidates: [0, nflushed) in the workspace list, the rest
// still in the wave's LDS stage.
struct SrcMain {
  const uint32_t* gk;
  const int32_t* gi;
  int nflushed;
  const uint2* stage;
  __device__ uint32_t key(int i) const { return i < nflushed ? gk[i] : stage[i - nflushed].x; }
  __device__ int32_t id(int i) const { return i < nflushed ? gi[i] : (int32_t)stage[i - nflushed].y; }
};

// ------------------------------------------------ key addressing

// Tile j of a row covers logical positions [64j, 64j+64).  A tile map gives
// the key index of the tile's first key (wave-uniform); the tile's keys are
// consecutive from there.
struct TileContig {
  __device__ int operator()(int tile) const { return tile << 6; }
};
// Paged cache with 64-token pages: tile j is page table[j] ("DSA TopK
// Indexer", contest report page: a page holds 64 tokens).
struct TilePaged {
  const int32_t* table;
  __device__ int operator()(int tile) const { return table[tile] << 6; }
};

// Id emitted for logical position i.
struct IdIdentity {
  __device__ int32_t operator()(int i) const { return i; }
};
struct IdPaged {
  const int32_t* table;
  __device__ int32_t operator()(int i) const { return table[i >> 6] * 64 + (i & 63); }
};

// Key index of logical position i under a tile map.
template <class TM>
__device__ __forceinline__ int key_index(const TM& tm, int i) { return tm(i >> 6) + (i & 63); }

// Threshold of one row from its sample lattice: positions s0 + OFFSET +
// stride*i, scored exactly like the main pass (same operations, so a
// sampled key reproduces its score bit for bit there); returns the r-th
// largest.  Whole workgroup calls; q is prepared by every wave.
template <class TM>
__device__ float sample_tau(const QOp& qo, const KeyBuf& kbuf, const TM& tm, int s0, const SampleGeom& sg,
                            uint32_t* s_samp, SelShared& sh, int tid) {
  const uint32_t lane = tid & 63;
  const int wave = tid >> 6;
  for (int tile = wave; tile * kTile < sg.n; tile += kWaves) {
    const int i0 = tile * kTile;
    const auto key_of = [&](int i) {
      const int smp = min(i0 + i, sg.n - 1);
      return key_index(tm, s0 + kSampleOffset + sg.stride * smp);
    };
    KeyTile kt;
    load_tile_gather(kt, kbuf, key_of, lane);
    const float sc = tile_score(qo, kt);
    const int i = i0 + (int)lane;
    if (i < sg.n) s_samp[i] = f2key(sc);
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

// Exact selection for one row without a threshold: rescore positions
// [s0, s1) into scratch (order-preserving keys), build the top-byte
// histogram on the way, finish the radix select over scratch and emit
// ids(i) of the winners into out[0..K).  Whole workgroup calls.
template <class TM, class IdMap>
__device__ void repair_row(const QOp& qo, const KeyBuf& kbuf, const TM& tm, const IdMap& ids, int s0, int s1,
                           int K, int32_t* out, uint32_t* scratch, SelShared& sh, int tid) {
  const uint32_t lane = tid & 63;
  const int wave = tid >> 6;
  const int L = s1 - s0, kr = L < K ? L : K;
  for (int i = tid; i < 256; i += kWG) sh.hist[i] = 0u;
  __syncthreads();
  const int tile_lo = s0 >> 6, tile_hi = (s1 + 63) >> 6;
  for (int tile = tile_lo + wave; tile < tile_hi; tile += kWaves) {
    KeyTile kt;
    load_tile(kt, kbuf, tm(tile), lane);
    const float sc = tile_score(qo, kt);
    const int my = (tile << 6) + (int)lane;
    const bool valid = my >= s0 && my < s1;
    const uint32_t key = f2key(sc);
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
