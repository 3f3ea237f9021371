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

// Candidates per row ("4.3 Candidate layout: warp-private segments" and "4.5
// Overflow spill area"): the main kernel splits each row's key tiles over S
// workgroups (parallelism along the keys for few rows, "10. The
// optimization target after fusion"), and each wave that walks a share of
// a row stores that share's candidates straight into a private workspace
// segment: nseg segments per row (see prefill_geom; the pages' on-chip
// store and spill area become one area in device memory).  The
// certificate's capacity per row is kCandCap (the default of the cand_cap
// test knob); a segment is sized so that a row short enough to keep all its
// keys (L <= kCandCap, threshold -inf) never overflows it, and a row also
// fails the certificate when one segment alone overflows.
// Largest y (and z) dimension of a launch grid: bounds the sequences of
// paged decode and the streams of the BF16 scan, which index it.
constexpr int kMaxGridY = 65535;

constexpr int kCandCap = 8192;
constexpr int kManyCands = 4096;  // rows keeping more are counted (idx_topk_stats.many_cands)
constexpr int kMaxSplit = 8;
constexpr int kSelRegs = 40;        // keys per thread of the select kernel, any nseg <= kMaxSeg
constexpr int kSelRegsFew = 33;     // ... for nseg <= 4 (seg_cap 8256, 4160, 2112 over 256, 128, 64 threads)
// Calls with at most kSelWideRows rows (one per CU) select each row with
// 1024 threads (a row's latency, not the CU's throughput, sets the time;
// at 512 rows the 256-thread select was faster), kSelRegsWide slots per
// thread for any nseg (seg_cap over 1024/nseg threads: at most 10).
constexpr int kSelWideRows = 256;
constexpr int kSelRegsWide = 10;

constexpr int kMaxSeg = kWaves * kMaxSplit;  // candidate segments per row, at most

// Geometry of the main kernel's walk.  One-pair walk: a workgroup takes
// one pair of rows and splits its tiles over its four waves and over S
// workgroups (S = 1, 2, 4, 8; nseg = kWaves * S segments per row).  Shared
// walk: a workgroup takes kSharedRows rows (a pair per wave), each tile is
// staged once in LDS for all four waves, and a row's candidates of one
// split go to one segment (S = 1, 2; nseg = S).
//
// Two workgroups per CU are resident (kRound in all), so a launch takes
// ceil(workgroups / kRound) rounds, and its time goes as rounds x (the
// tiles one workgroup walks + its prologue, about kWgFixed tiles' worth).
// Each split samples its rows again (about 2% per extra split), and the
// shared walk does its work about 5% faster (its tiles come from LDS; 3.26
// against 3.46 ms at 4096 x 131072) with four times coarser workgroups.  The
// geometry of lowest cost is taken, the shared walk only from
// kSharedMinRows rows.  Measured at 131072 keys, ms per call, shared against
// one-pair: 2048 rows 1.72 against 1.80, 3072 rows 2.95 against 2.58 (the
// shared walk's 768 workgroups fill 1.5 rounds), 4096 rows 3.26 against
// 3.46; the cost picks the faster walk at 2560, 3584, 5120 and 6144 rows.
constexpr int kSharedRows = 2 * kWaves;
constexpr int kSharedMinRows = 2048;
constexpr int kRound = 512;
constexpr int kWgFixed = 8;

struct WalkGeom {
  int shared, S, nseg;
};

__host__ __device__ inline int64_t walk_rounds(int64_t wgs) { return (wgs + kRound - 1) / kRound; }

// rounds x (pair-tiles per workgroup + prologue) x (1 + 2% per extra split)
// x (20 for the one-pair walk, 19 for the shared walk)
__host__ __device__ inline int64_t walk_cost(int64_t wgs, int64_t pair_tiles, int s, int walk) {
  return walk_rounds(wgs) * (pair_tiles + kWgFixed) * (50 + s - 1) * walk;
}

__host__ __device__ inline WalkGeom prefill_geom(int rows, int nkeys) {
  const int64_t tiles = nkeys > 0 ? ((int64_t)nkeys + 63) / 64 : 1;
  const int64_t pairs = (rows + 1) / 2, groups = (rows + kSharedRows - 1) / kSharedRows;
  WalkGeom best{0, 1, kWaves};
  int64_t best_cost = walk_cost(pairs, tiles, 1, 20);
  for (int s = 2; s <= kMaxSplit; s *= 2) {
    const int64_t c = walk_cost(pairs * s, (tiles + s - 1) / s, s, 20);
    if (c < best_cost) {
      best_cost = c;
      best = WalkGeom{0, s, kWaves * s};
    }
  }
  if (rows >= kSharedMinRows) {
    for (int s = 1; s <= 2; s *= 2) {
      const int64_t c = walk_cost(groups * s, (4 * tiles + s - 1) / s, s, 19);
      if (c < best_cost) {
        best_cost = c;
        best = WalkGeom{1, s, s};
      }
    }
  }
  return best;
}

// Entries of one candidate segment for nseg segments per row: the larger of
// an even share of kCandCap and the tiles an unaligned kCandCap-key row
// puts on one segment (such a row spans kCandCap/64 + 1 tiles).
__host__ __device__ inline int prefill_seg_cap(int nseg) {
  const int share = kCandCap / nseg;
  const int tiles = (kCandCap / 64 + 1 + nseg - 1) / nseg;
  return share > tiles * 64 ? share : tiles * 64;
}

// Exact repair, split over the chip: one work item covers kRepairChunk
// positions of one failed row; scratch holds the scores of up to
// repair_slots() failed rows at once, and kRepairFallback more slots serve
// workgroups that repair whole rows alone once the slots run out.
constexpr int kRepairChunk = 4096;
constexpr int kRepairGrid = 256;  // one workgroup per CU; items are strided over the grid
constexpr int kRepairPassGrid = 1024;  // digit pass and gather: four workgroups per CU
constexpr int kRepairWalkWGs = 512;    // rescoring walk: the workgroups of one round, two per CU
// The chip-wide passes resolve the top two 8-bit digits of the K-th key;
// the keys that share them with it (the boundary group) are gathered into
// the failed row's candidate area, which the fast path no longer needs, and
// one workgroup per row selects among them in registers.  A larger group
// (massive ties) is selected by that workgroup from the row's scratch.
constexpr int kRepairDigits = 2;
constexpr int kRepairGroupCap = kCandCap;  // gathered boundary keys per row (<= its candidate area)
constexpr int kRepairFinalGrid = 256;  // workgroups of 1024 threads, one row each at a time

// Words kept per slotted repair row (PrefillArgs::rrow): the gather's
// output counters (keys above the boundary emitted; boundary keys emitted
// or gathered), then two groups of four holding the row's selection state
// after one and after two digits (prefix, mask, rem, and the size of the
// boundary group or 0xFFFFFFFF once that group is taken whole: every key
// with (key & mask) > prefix is taken, and rem more among those equal to
// it).
constexpr int kRowGt = 0, kRowEq = 1, kRowState = 4;
constexpr int kRowWords = 12;
constexpr int kRepairFallback = 256;
constexpr int64_t kRepairScratchKeys = (int64_t)1 << 28;  // 1 GiB of scores

// Control words at the start of every workspace: the failure count, then
// kStatLanes copies of the idx_topk_stats counters, one 128-byte line each
// (workgroup b counts into copy b % kStatLanes, so that thousands of
// per-row increments do not queue on one address; the reader sums them).
constexpr int kCtrlFail = 0;   // number of rows on the failure list
constexpr int kStatsOff = 32;  // first counter copy
constexpr int kStatLanes = 32;
constexpr int kStatStride = 32;  // words between copies
constexpr int kStatCount = 8;    // counters per copy, idx_topk_stats order
constexpr int kCtrlWords = kStatsOff + kStatLanes * kStatStride;
constexpr int kStRows = 0, kStFast = 1, kStUnder = 2, kStOver = 3, kStMany = 4,
              kStRepaired = 5, kStTrivial = 6, kStBad = 7;

__device__ __forceinline__ uint32_t* stat_copy(uint32_t* ctrl, int block) {
  return ctrl + kStatsOff + (block & (kStatLanes - 1)) * kStatStride;
}

// Zero the control words (first workgroup of the first kernel of a call).
__device__ __forceinline__ void clear_ctrl(uint32_t* ctrl, int tid) {
  for (int i = tid; i < kCtrlWords; i += kWG) ctrl[i] = 0u;
}

// Scratch row stride (keys): N rounded up to 64, so rows are 256-byte aligned.
__host__ __device__ inline int64_t repair_stride(int nkeys) { return ((int64_t)nkeys + 63) & ~(int64_t)63; }

// Failed rows whose scores fit the repair scratch together: at most
// kRepairScratchKeys scores, at least kRepairFallback rows, at most Q.
__host__ __device__ inline int repair_slots(int rows, int nkeys) {
  const int64_t ns = repair_stride(nkeys);
  int64_t s = ns > 0 ? kRepairScratchKeys / ns : (int64_t)rows;
  if (s < kRepairFallback) s = kRepairFallback;
  if (s > rows) s = rows;
  return s > 0 ? (int)s : 1;
}

// Scratch rows in all: the slots plus, when some rows may not get a slot,
// the fallback workgroups' own rows.
__host__ __device__ inline int repair_rows(int rows, int nkeys) {
  const int s = repair_slots(rows, nkeys);
  return s + (rows > s ? kRepairFallback : 0);
}

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
  uint2* cand;          // [Q][nseg][seg_cap] candidates: (FP32 score bits, key id)
  uint32_t* segn;       // [Q][nseg][4]: entries stored, key of the largest dropped candidate
                        // (0: none), position of the first dropped one, unused
  int32_t S, seg_cap, seg_eff;  // splits, segment stride, usable entries per segment
  int32_t shared, nseg;         // shared walk (kSharedRows rows per workgroup); segments per row
  int32_t cand_cap;  // candidates stored per row (the certificate's capacity)
  int32_t* fail_list;   // [Q]
  uint32_t* ctrl;       // kCtrlWords
  uint32_t* scratch;    // [repair_rows][repair_stride(N)] repair scores (order-preserving keys)
  uint32_t* rhist;      // [rslots][kRepairDigits][256] digit histograms of each slotted repair row
  uint32_t* rrow;       // [rslots][kRowWords] counters and selection state of each slotted repair row
  int32_t rslots;
  int64_t rstride;
  float* dbg_scores;    // [Q][N] or null
  int32_t* row_status;  // [Q] or null: IDX_ROW_* outcome of each row
  uint64_t* clock;      // [2] or null: summed shader-clock cycles and wall-clock ticks of the main kernel's waves
  int32_t math_only;    // control build: scores folded into checksums, no filter and no selection
  int32_t force_tau;
  int32_t keep_all;  // every valid row keeps all its keys (N <= kCandCap): no sampler, no repair
  int32_t fuse_tau;  // one split: the main kernel takes its rows' thresholds itself
  int32_t direct;    // no relaid copy: the one-pair walk (and the repair) read key tiles from k
                     // itself, as the shared walk always does
  int32_t clear_main;  // no kernel ran before the main one: it clears the counters and repair state
  float tau_value;
  hipEvent_t ev_main_start, ev_main_stop;  // host-side only: timing hooks
  int32_t main_reps;                       // host-side only: launches of the main kernel
};

struct SampleGeom {
  int n, stride, r;
};

// Sample lattice of a row of length L: positions OFFSET + stride*i < L.  Rows
// that fit the candidate capacity need no threshold (n = 0: tau = -inf).
__device__ inline SampleGeom sample_geom(int L, int cand_cap) {
  SampleGeom g{0, kSampleStride, 0};
  if (L <= cand_cap || L <= kSampleOffset) return g;
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

// ------------------------------------------------ key addressing

// Tile j of a row covers logical positions [64j, 64j+64).  A tile map gives
// the key index of the tile's first key (wave-uniform); the tile's keys are
// consecutive from there.
struct TileContig {
  __device__ int operator()(int tile) const { return tile << 6; }
};
// Paged cache with 64-token pages: tile j is page table[j] ("DSA TopK
// Indexer", contest report page (arXiv 2608.14560): a page holds 64 tokens).
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
  int32_t npages;  // the page index is clamped to [0, npages): an unused register slot (any id) reads a real entry
  __device__ int32_t operator()(int i) const { return table[min(max(i >> 6, 0), npages - 1)] * 64 + (i & 63); }
};

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
  const SelResult sel = (L > kr) ? radix_select(src, L, kr, sh, tid, true, true) : SelResult{0u, 0u, kr, kr};
  emit_selection(src, L, sel, kr, K, out, sh, tid);
}

int launch_prefill(const PrefillArgs& A, hipStream_t stream);
int launch_prefill_unfused(const PrefillArgs& A, hipStream_t stream);

}  // namespace idxk
