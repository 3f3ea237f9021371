// Exact top-K over a dense FP32 score matrix, one workgroup per row: the
// standalone selection stage of an unfused pipeline (Fusing Indexer Scoring
// and Exact Top-k page, "2.2 Indexer scoring is compute-bound": score into an
// explicit [Q,N] matrix, then select; "3.5 Stage result", Table 2: the
// standalone top-k), kept as the comparator for the fused path, as the
// selection stage of the paged decode, and as a library routine of its own.
//
// Per row of length L > K:
//   0. a cut c from a sample of the row: kSampleKeys scores in contiguous
//      blocks of one score per thread spread over it, c = a sample key with
//      about 2K of the row's keys expected at or above it (the page's
//      sampled threshold, "3.2 Sampled threshold", applied to an explicit
//      score row);
//   1. one streaming pass gathers every key >= c into LDS (a row shorter
//      than the sample, c = key 0: all of it), each wave into a private
//      segment with a scalar count; with K to kRowsCap of them, the
//      register-resident range select over the gathered keys finishes the
//      row (ties at the K-th score to the lowest ids): one read of the row.
// Otherwise (a cut that kept too few or too many keys) two more passes: a 2048-bin histogram of the top 11 bits
// of the order-preserving keys (>= c when c kept too many) finds the bin b
// of the K-th largest key ("3.2": radix select on order-preserving 32-bit
// integers); the next pass writes out every key in a bin above b and
// gathers bin b, which the range select finishes.  A bin too large for LDS
// (massive ties) goes to the generic four-digit radix select over the row
// in memory, with the same tie rule.
#include <type_traits>

#include "idx_internal.hpp"

#include "idx_rows.hpp"

namespace idxk {

constexpr int kRowsBins = 2048;
constexpr int kRowsShift = 21;  // 32 - 11 bits
constexpr int kRowsCap = 6144;  // gathered keys held in LDS
constexpr int kSampleKeys = 4096;  // sample: kSampleKeys / NT blocks of NT scores
constexpr int kSampleMinLen = kSampleKeys;  // shorter rows (< kRowsCap keys) are gathered whole
constexpr int kDecodeRegs = 8;  // register slots per thread for a decode row's filtered candidates
// Per workgroup size (NW waves, NT threads): register slots of the
// gathered list, each wave's private gather segment, sample blocks.
template <int NW>
struct RowsGeom {
  static constexpr int NT = 64 * NW;
  static constexpr int Regs = kRowsCap / NT;
  static constexpr int SegCap = kRowsCap / NW;
  static constexpr int SampleBlocks = kSampleKeys / NT;
};
constexpr int kSampleBlocks = RowsGeom<kWaves>::SampleBlocks;

// Dense row in memory: element i is position s0 + i, emitted as ids(s0 + i).
template <class IdMap>
struct SrcDense {
  const float* row;
  int32_t s0;
  IdMap ids;
  __device__ uint32_t key(int i) const { return f2key(row[i]); }
  __device__ int32_t id(int i) const { return ids(s0 + i); }
};

// Calls f(i, valid, key) for every element i < L of the row (and for some
// positions outside it with valid = false), reading it with 16-byte buffer
// loads from the 16-byte-aligned address at or below the row's start (reads
// past the end return 0), U loads per thread per step; the next step's
// loads are issued before this step's keys are processed.
template <int U, int NW = kWaves, class F>
__device__ __forceinline__ void for_each_key(const float* row, int L, int tid, const F& f) {
  constexpr int kRowsUnroll = U;
  constexpr int NT = 64 * NW;
  const int shift = (int)(((uintptr_t)row & 15u) >> 2);  // elements before the row in its first 16 bytes
  const float* abase = row - shift;
  const int span = L + shift;
  const rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, span * 4, 0x00020000);
  constexpr int kStep = NT * 4 * kRowsUnroll;
  const auto load = [&](v4i (&v)[kRowsUnroll], int base) {
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rr, (base + (u * NT + tid) * 4) * 4, 0, 0);
  };
  const auto process = [&](const v4i (&v)[kRowsUnroll], int base) {
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
      const int i0 = base + (u * NT + tid) * 4 - shift;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        f(i, i >= 0 && i < L, f2key(__int_as_float(v[u][e])));
      }
    }
  };
  // two buffers in turn, no copy between them: a register copy of a load's
  // result would wait for that load (the memory counter retires in order)
  v4i a[kRowsUnroll], b[kRowsUnroll];
  load(a, 0);
  for (int base = 0; base < span; base += 2 * kStep) {
    load(b, base + kStep);
    process(a, base);
    load(a, base + 2 * kStep);
    process(b, base + kStep);
  }
}

// Gathers the keys >= cut of the row into this wave's segment (lkey/lid
// point at it, SegCap entries) and returns how many there were (more than
// SegCap: the excess was not stored).  Same loads as for_each_key; per
// step each thread counts its qualifying keys, a wave scan turns the counts
// into slots after the wave's running total, and each thread stores its
// keys there: vector instructions only, no branch or atomic per key.
template <int U, int NW = kWaves>
__device__ __forceinline__ uint32_t gather_ge(const float* row, int L, int tid, uint32_t cut, uint32_t* lkey,
                                              int32_t* lid, int32_t s0) {
  constexpr int NT = 64 * NW;
  constexpr uint32_t kSegCap = (uint32_t)RowsGeom<NW>::SegCap;
  const uint32_t lane = tid & 63;
  const int shift = (int)(((uintptr_t)row & 15u) >> 2);
  const float* abase = row - shift;
  const int span = L + shift;
  const rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, span * 4, 0x00020000);
  constexpr int kStep = NT * 4 * U;
  const auto load = [&](v4i (&v)[U], int base) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rr, (base + (u * NT + tid) * 4) * 4, 0, 0);
  };
  const auto take = [&](int i, int v) { return i >= 0 && i < L && f2key(__int_as_float(v)) >= cut; };
  uint32_t wcnt = 0u;
  const auto step = [&](const v4i (&cur)[U], int base) {
    uint32_t cnt = 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i0 = base + (u * NT + tid) * 4 - shift;
#pragma unroll
      for (int e = 0; e < 4; ++e) cnt += take(i0 + e, cur[u][e]) ? 1u : 0u;
    }
    const uint32_t inc = wave_inclusive_sum(cnt);  // inclusive scan over the wave's lanes
    uint32_t slot = wcnt + inc - cnt;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i0 = base + (u * NT + tid) * 4 - shift;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool g = take(i0 + e, cur[u][e]);
        if (g && slot < kSegCap) {
          lkey[slot] = f2key(__int_as_float(cur[u][e]));
          lid[slot] = s0 + i0 + e;
        }
        slot += g ? 1u : 0u;
      }
    }
    wcnt += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  };
  v4i a[U], b[U];  // in turn, no copy between them (see for_each_key)
  load(a, 0);
  for (int base = 0; base < span; base += 2 * kStep) {
    load(b, base + kStep);
    step(a, base);
    load(a, base + 2 * kStep);
    step(b, base + kStep);
  }
  return wcnt;
}

struct RowsShared {
  union {
    uint32_t hist[kRowsBins];  // histogram path, before the gather
    uint32_t lkey[kRowsCap];
  };
  int32_t lid[kRowsCap];
  uint32_t n_gt, n_eq, bin, above, inbin, pad[3];
  uint32_t segc[kMaxWaves];  // keys each wave's gather segment received
  SelShared sh;
};

// Step 0: the sampled cut of a row of length L > K (key 0 keeps every key):
// the r-th largest of kSampleKeys sampled keys, r chosen so that about 2K
// of the row's keys are expected at or above it.  All threads call this.
// Split in two so that a caller can issue other loads between them: the
// sample's loads (L >= 1; indexes clamped, so a short row reads valid
// elements whose keys then go unused) and its select.
template <int NW = kWaves>
__device__ __forceinline__ void sample_load(const float* row, int L, uint32_t (&sk)[RowsGeom<NW>::SampleBlocks],
                                            int tid) {
  constexpr int SB = RowsGeom<NW>::SampleBlocks, NT = 64 * NW;
  const int step = max(0, (L - NT) / (SB - 1));  // block j starts at j*step
#pragma unroll
  for (int j = 0; j < SB; ++j) sk[j] = f2key(row[min(j * step + tid, L - 1)]);
}

template <int NW = kWaves>
__device__ __forceinline__ uint32_t sample_select(const uint32_t (&sk)[RowsGeom<NW>::SampleBlocks], int L, int K,
                                                  SelShared& sh, int tid) {
  constexpr int SB = RowsGeom<NW>::SampleBlocks;
  if (L < kSampleMinLen) return 0u;
  // rank r in the sample <=> about r * L / kSampleKeys keys of the row
  const int r = (int)(((int64_t)2 * K * kSampleKeys + L - 1) / L);
  if (r >= kSampleKeys) return 0u;
  const RegLayout lay{(uint32_t)tid, (uint32_t)(64 * NW), (uint32_t)kSampleKeys, (uint32_t)SB};
  return range_select_regs<SB, NW>([&](int j) { return sk[j]; }, lay, r, sh, tid).lo;
}

template <int NW = kWaves>
__device__ __forceinline__ uint32_t sample_cut(const float* row, int L, int K, SelShared& sh, int tid) {
  if (L < kSampleMinLen) return 0u;
  uint32_t sk[RowsGeom<NW>::SampleBlocks];
  sample_load<NW>(row, L, sk, tid);
  return sample_select<NW>(sk, L, K, sh, tid);
}

// Exact selection of the rem largest of the gathered keys (ties to the
// lowest positions), ids(position) written to out[0, rem).  The keys sit in
// NW segments of lkey/lid: segment w holds c[w] keys from w*stride (the
// histogram path passes one segment).  1 <= rem <= n = sum of c[w] <=
// kRowsCap.  All threads call this.
template <int NW, class IdMap>
__device__ __forceinline__ void select_gathered(RowsShared& S, const uint32_t (&c)[NW], uint32_t stride,
                                                int rem, int32_t* out, const IdMap& ids, int tid) {
  constexpr int Regs = RowsGeom<NW>::Regs;
  uint32_t n = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) n += c[w];
  const RegLayout lay = block_list_layout<NW>(n, (uint32_t)tid);
  uint32_t key[Regs];
  int32_t id[Regs];
#pragma unroll
  for (int j = 0; j < Regs; ++j) {
    uint32_t x = lay.at(j), at = x;  // list element x -> its segment slot
    bool later = true;               // x lies beyond the segments seen so far
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) {
      later = later && x >= c[w];
      x = later ? x - c[w] : x;
      at = later ? x + (uint32_t)(w + 1) * stride : at;
    }
    const bool v = lay.valid(j);
    key[j] = v ? S.lkey[at] : 0u;
    id[j] = v ? S.lid[at] : 0;
  }
  const auto kf = [&](int j) { return key[j]; };
  const RangeSel sel = (n > (uint32_t)rem) ? range_select_regs<Regs, NW>(kf, lay, rem, S.sh, tid)
                                            : RangeSel{1u, 0xFFFFFFFFu, rem, (int)n};
  const uint32_t idlo = tie_bound_regs<NW>(key, id, lay, sel, S.sh, tid);
  emit_range_regs<NW>(key, id, lay, sel, idlo, rem, rem, out, ids, S.sh, tid);
}

// Rows of a dense matrix: row t is scores + t*ld, range [row_start[t],
// row_end[t]) (row_start null: [0, row_end[t])), ids are positions.
struct DenseRows {
  template <int NW>
  static constexpr int unroll() { return 4; }  // many rows: workgroups enough to cover the latency
  static constexpr int kMinBlocks = 3;
  RowsArgs A;
  template <int NW>
  __device__ __forceinline__ bool range(int t, int& s0, int& s1, int) const {
    s0 = A.row_start ? A.row_start[t] : 0;
    s1 = A.row_end[t];
    return s0 >= 0 && s0 <= s1 && s1 <= A.N;
  }
  // the pre-gather's check (the same)
  __device__ __forceinline__ bool gather_range(int t, int& s0, int& s1, int tid) const {
    return range<kWaves>(t, s0, s1, tid);
  }
  __device__ __forceinline__ const float* row(int t) const { return A.scores + (int64_t)t * A.ld; }
  __device__ __forceinline__ IdIdentity ids(int) const { return IdIdentity{}; }
};

// Sequences of the paged decode: row b holds the scores of logical positions
// [0, seq_lens[b]) at scores + b*ld; it is invalid when its length is out of
// range or one of the page ids it uses is outside [0, num_pages) (checked
// here, by the selection); ids are physical cache slots.
struct PagedRows {
  // few long rows: one workgroup must cover the latency alone (four times
  // fewer loads per step with four times the threads)
  template <int NW>
  static constexpr int unroll() { return NW >= 16 ? 4 : 16; }
  static constexpr int kMinBlocks = 1;
  RowsArgs A;
  // all threads call this: the length and every page id the sequence uses,
  // four loads per thread in flight per round of 4*NT pages (clamped
  // indexes, no branch per load), then a workgroup OR
  template <int NW>
  __device__ __forceinline__ bool range(int b, int& s0, int& s1, int tid) const {
    constexpr int NT = 64 * NW;
    s0 = 0;
    s1 = A.row_end[b];
    bool bad = s1 < 0 || s1 > A.N;
    const int np = bad ? 0 : (s1 + 63) >> 6;
    const int32_t* pt = A.table + (int64_t)b * A.max_pages;
    for (int p0 = 0; p0 < np; p0 += 4 * NT) {
      int pg[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) pg[u] = pt[min(p0 + u * NT + tid, np - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) bad |= (p0 + u * NT + tid < np) & ((pg[u] < 0) | (pg[u] >= A.num_pages));
    }
    return !__syncthreads_or(bad);
  }
  // the pre-gather checks the length only: the page ids decide the output,
  // which the select kernel writes (-1 for a bad sequence), not what is gathered
  __device__ __forceinline__ bool gather_range(int b, int& s0, int& s1, int) const {
    s0 = 0;
    s1 = A.row_end[b];
    return s1 >= 0 && s1 <= A.N;
  }
  __device__ __forceinline__ const float* row(int b) const { return A.scores + (int64_t)b * A.ld; }
  __device__ __forceinline__ IdPaged ids(int b) const { return IdPaged{A.table + (int64_t)b * A.max_pages, A.max_pages}; }
};

// Dense rows come by the thousand: three 256-thread workgroups per CU (LDS
// allows three) keep enough loads in flight.  Paged decode rows are few and
// long: one workgroup per row with no occupancy bound, so that the register
// select does not spill, and 1024 threads (NW = 16), whose shorter per-thread
// chains select a sequence's candidates faster (13 against 15 us for 16
// sequences' pre-gathered keys); reading and selecting a whole sequence in
// that one workgroup took 30 us.
template <class Rows, int NW>
__global__ __launch_bounds__(64 * NW, Rows::kMinBlocks) void k_topk_rows(RowsArgs A) {
  constexpr int NT = 64 * NW;
  constexpr int Regs = RowsGeom<NW>::Regs;
  constexpr int SegCap = RowsGeom<NW>::SegCap;
  constexpr int U = Rows::template unroll<NW>();
  __shared__ RowsShared S;
  const Rows R{A};
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  int32_t* out = A.out + (int64_t)t * A.K;
  uint32_t* stats = A.ctrl ? stat_copy(A.ctrl, blockIdx.x) : nullptr;
  if (stats && tid == 0) atomicAdd(&stats[kStRows], 1u);
  // pre-gathered regions: every slot this thread may hold and the region's
  // count, loaded first (their addresses depend on neither the count nor
  // the row's checks), so that they arrive with the range check's loads
  // instead of two round trips after it.  Region g is read by the NT/G
  // threads g*NT/G .. ; thread slot j holds region element
  // (tid mod NT/G) + j*NT/G.
  uint32_t graw[Regs];
  int32_t iraw[Regs];
  uint32_t gc = 0u;
  if (A.gcnt) {
    const int G = A.gsplit;  // a power of two <= kMaxGatherSplit
    const uint32_t tpr = (uint32_t)(NT / G);
    const int g = tid / (int)tpr;
    const int64_t region = ((int64_t)t * G + g) * A.gcap;
#pragma unroll
    for (int j = 0; j < Regs; ++j) {
      const int64_t e = region + min((uint32_t)tid % tpr + (uint32_t)j * tpr, (uint32_t)A.gcap - 1u);
      graw[j] = A.gkey[e];
      iraw[j] = A.gid[e];
    }
    gc = A.gcnt[(int64_t)t * G + g];
  }
  // the scoring kernel's plan for this row (filtered decode candidates),
  // loaded beside the range check; only used for a row it scored
  uint2 dpl = make_uint2(0u, 0u);
  uint2 dc2 = make_uint2(0u, 0u);  // counts of segments 2 tid and 2 tid + 1 (valid below 4 dpl.y)
  if (A.dcnt) {
    dpl = A.dplan[t];
    dc2 = reinterpret_cast<const uint2*>(A.dcnt + (int64_t)t * kDecodeCntStride)[min(tid, kDecodeCntStride / 2 - 1)];
  }
  int s0, s1;
  if (!R.template range<NW>(t, s0, s1, tid)) {
    for (int i = tid; i < A.K; i += NT) out[i] = -1;
    if (stats && tid == 0) atomicAdd(&stats[kStBad], 1u);
    return;
  }
  const int L = s1 - s0;
  const int K = A.K;
  const auto ids = R.ids(t);
  if (L <= K) {  // every key of the row, in position order
    for (int i = tid; i < K; i += NT) out[i] = i < L ? ids(s0 + i) : -1;
    if (stats && tid == 0) atomicAdd(&stats[kStTrivial], 1u);
    return;
  }
  const float* row = R.row(t) + s0;

  // pre-gathered regions that hold K to kRowsCap keys in all and each fit
  // its threads' registers: select from them
  if (A.gcnt) {
    const int G = A.gsplit;
    const uint32_t tpr = (uint32_t)(NT / G);
    uint32_t n = 0u;
    block_exclusive_scan<NW>(tid % (int)tpr == 0 ? gc : 0u, S.sh, tid, n);
    const bool fits = !__syncthreads_or(gc > tpr * (uint32_t)Regs);
    if (fits && n >= (uint32_t)K) {
      // slots past the wave's fullest region are empty in all its threads
      uint32_t jw = (gc + tpr - 1u) / tpr;
      jw = wave_max_u32(jw);
      const RegLayout lay{(uint32_t)tid % tpr, tpr, gc, jw};
      uint32_t key[Regs];
      int32_t id[Regs];
#pragma unroll
      for (int j = 0; j < Regs; ++j) {
        const bool v = lay.valid(j);
        key[j] = v ? graw[j] : 0u;
        id[j] = v ? iraw[j] : 0;
      }
      const auto kf = [&](int j) { return key[j]; };
      const RangeSel sel = (n > (uint32_t)K) ? range_select_regs<Regs, NW>(kf, lay, K, S.sh, tid)
                                              : RangeSel{1u, 0xFFFFFFFFu, K, (int)n};
      const uint32_t idlo = tie_bound_regs<NW>(key, id, lay, sel, S.sh, tid);
      emit_range_regs<NW>(key, id, lay, sel, idlo, K, K, out, ids, S.sh, tid);
      if (stats && tid == 0) atomicAdd(&stats[kStFast], 1u);
      return;
    }
  }

  // candidates filtered by the scoring kernel: all of the row's keys at or
  // above its threshold, in the four wave segments of each of the row's
  // dpl.y workgroups.  The segments' counts (two per thread) are scanned
  // into offsets of one list (in LDS), whose element x thread slot j of
  // thread x mod NT holds (x = tid + j*NT); the segment of x is found by a
  // binary search over the offsets.  A segment that dropped candidates
  // enters the scan as more than the slots hold, so one total tells both.
  // Exact when every segment kept all its candidates, they fit the slots
  // and there are at least K of them (every other key scores below the
  // threshold); otherwise the row takes the passes below.
  if (2 * NT >= kDecodeCntStride && A.dcnt) {  // two counts per thread cover the row's (paged rows)
    constexpr int DR = kDecodeRegs;
    const int nseg = 4 * (int)dpl.y;  // at most 2048 (512 workgroups)
    const int64_t seg0 = (int64_t)dpl.x * kWaves;
    const uint32_t ca = 2 * tid < nseg ? dc2.x : 0u, cb = 2 * tid + 1 < nseg ? dc2.y : 0u;
    const bool over = ca > (uint32_t)A.dseg || cb > (uint32_t)A.dseg;
    uint32_t n = 0u;
    const uint32_t pa = block_exclusive_scan<NW>(over ? (uint32_t)(NT * DR + 1) : ca + cb, S.sh, tid, n);
    uint32_t* const off = S.lkey;  // nseg + 1 offsets (the LDS list area is unused on this path)
    if (2 * tid < nseg) off[2 * tid] = pa;
    if (2 * tid + 1 < nseg) off[2 * tid + 1] = pa + ca;
    if (tid == 0) off[nseg] = n;
    __syncthreads();
    const bool dropped = n > (uint32_t)(NT * DR);
    if (nseg >= 1 && !dropped && n >= (uint32_t)K) {
      const RegLayout lay = block_list_layout<NW>(n, (uint32_t)tid);
      uint32_t sg[DR], lo[DR];  // per slot: search window [lo, lo + span)
#pragma unroll
      for (int j = 0; j < DR; ++j) lo[j] = 0u;
      for (int span = nseg; span > 1;) {  // largest segment s with off[s] <= x
        const int half = span >> 1;
#pragma unroll
        for (int j = 0; j < DR; ++j) {
          const uint32_t mid = lo[j] + (uint32_t)half;
          lo[j] = off[mid] <= lay.at(j) ? mid : lo[j];
        }
        span -= half;
      }
      uint32_t key[DR];
      int32_t id[DR];
#pragma unroll
      for (int j = 0; j < DR; ++j) {
        const bool ok = lay.valid(j);
        sg[j] = lo[j];
        const uint2 pr = ok ? A.dcand[(seg0 + sg[j]) * A.dseg + (lay.at(j) - off[sg[j]])] : make_uint2(0u, 0u);
        key[j] = pr.x;
        id[j] = (int32_t)pr.y;
      }
      const auto kf = [&](int j) { return key[j]; };
      const RangeSel sel = (n > (uint32_t)K) ? range_select_regs<DR, NW>(kf, lay, K, S.sh, tid)
                                              : RangeSel{1u, 0xFFFFFFFFu, K, (int)n};
      const uint32_t idlo = tie_bound_regs<NW>(key, id, lay, sel, S.sh, tid);
      emit_range_regs<NW>(key, id, lay, sel, idlo, K, K, out, ids, S.sh, tid);
      if (stats && tid == 0) atomicAdd(&stats[kStFast], 1u);
      return;
    }
    // the candidates do not settle the row: counted as an overflow (some
    // were dropped) or an underflow (fewer than K), then the passes below
    if (stats && tid == 0) atomicAdd(&stats[dropped ? kStOver : kStUnder], 1u);
    __syncthreads();  // the offsets' LDS is the passes' list area
  }

  // step 0: the sampled cut (key 0 keeps every key)
  uint32_t cut = sample_cut<NW>(row, L, K, S.sh, tid);

  // step 1: one pass gathering the keys at or above the cut into the
  // waves' private segments (slot = the wave's scalar count + rank in the
  // ballot: no atomics)
  uint32_t c[NW];  // keys in each segment
#pragma unroll
  for (int w = 0; w < NW; ++w) c[w] = 0u;
  uint32_t stride = (uint32_t)SegCap;
  int rem = K;       // how many of them to take
  int32_t* dst = out;
  bool gathered = false;
  {
    const int wave = tid >> 6;
    const uint32_t wcnt = gather_ge<U, NW>(row, L, tid, cut, S.lkey + wave * SegCap, S.lid + wave * SegCap, s0);
    if ((tid & 63) == 0) S.segc[wave] = wcnt;
    __syncthreads();
    uint32_t n = 0u;
    bool full = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      c[w] = S.segc[w];
      n += c[w];
      full |= c[w] > (uint32_t)SegCap;
    }
    gathered = n >= (uint32_t)K && !full;
    if (n < (uint32_t)K) cut = 0u;  // the cut kept too few keys: histogram the whole row
    __syncthreads();
  }
  static_assert(kSampleMinLen <= kRowsCap, "unsampled rows must fit the gather");

  bool generic = false;  // the boundary bin does not fit in LDS
  if (!gathered) {
    // histogram path: the bin of the K-th largest key among keys >= cut
    for (int i = tid; i < kRowsBins; i += NT) S.hist[i] = 0u;
    if (tid == 0) { S.n_gt = 0u; S.n_eq = 0u; }
    __syncthreads();
    for_each_key<U, NW>(row, L, tid, [&](int, bool v, uint32_t key) {
      hist_add(S.hist, key >> kRowsShift, v && key >= cut);  // returns at once when no lane qualifies
    });
    __syncthreads();
    {
      // thread u holds bins BPT*u .. BPT*u + BPT-1
      constexpr int BPT = kRowsBins / NT;
      uint32_t h[BPT], a = 0u;
#pragma unroll
      for (int j = 0; j < BPT; ++j) { h[j] = S.hist[BPT * tid + j]; a += h[j]; }
      uint32_t total;
      const uint32_t before = block_exclusive_scan<NW>(a, S.sh, tid, total);
      uint32_t ab = total - before - a;  // keys in bins above this thread's
      const uint32_t r = (uint32_t)K;
      if (ab < r && r <= ab + a) {
#pragma unroll
        for (int j = BPT - 1; j >= 0; --j) {
          if (ab < r && r <= ab + h[j]) { S.bin = (uint32_t)(BPT * tid + j); S.above = ab; S.inbin = h[j]; }
          ab += h[j];
        }
      }
    }
    __syncthreads();
    const uint32_t bin = S.bin, above = S.above, inbin = S.inbin;

    // keys above the bin go straight out; the bin's keys (>= cut) to LDS
    for_each_key<U, NW>(row, L, tid, [&](int i, bool v, uint32_t key) {
      const uint32_t d = key >> kRowsShift;
      const bool gt = v && d > bin, eq = v && d == bin && key >= cut;
      if (__ballot(gt || eq)) {
        const uint32_t pg = reserve(&S.n_gt, gt);
        if (gt) out[pg] = ids(s0 + i);
        const uint32_t pe = reserve(&S.n_eq, eq);
        if (eq && pe < (uint32_t)kRowsCap) { S.lkey[pe] = key; S.lid[pe] = s0 + i; }
      }
    });
    __syncthreads();
    c[0] = inbin;
#pragma unroll
    for (int w = 1; w < NW; ++w) c[w] = 0u;
    stride = 0u;
    rem = K - (int)above;  // 1 <= rem <= inbin
    dst = out + above;
    generic = inbin > (uint32_t)kRowsCap;
  }

  if (!generic) {
    select_gathered<NW>(S, c, stride, rem, dst, ids, tid);
    if (stats && tid == 0) atomicAdd(&stats[kStFast], 1u);
  } else {
    // the bin does not fit: exact radix select over the row in memory
    const SrcDense<decltype(ids)> src{row, s0, ids};
    const SelResult sel = radix_select<NW>(src, L, K, S.sh, tid, false, true);
    emit_selection<NW>(src, L, sel, K, K, out, S.sh, tid);
    if (stats && tid == 0) atomicAdd(&stats[kStRepaired], 1u);
  }
}

// Pre-gather of long rows (scan streams; paged decode sequences of batches
// beyond 256, whose scoring kernel does not filter): workgroup
// (g, t) computes row t's sampled cut (as the per-row kernel would) and
// stores the keys >= cut of slice g of the row into its own region of the
// workspace; each thread counts its keys, one workgroup scan gives the
// slots, with no atomics (same-address device atomics from every
// workgroup of a row would queue at one L2 line).  Spreads over many CUs
// the pass that one workgroup per row would make alone.
template <class Rows>
__global__ __launch_bounds__(kWG) void k_rows_gather(RowsArgs A) {
  __shared__ SelShared sh;
  const Rows R{A};
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int g = blockIdx.x, t = blockIdx.y;
  int s0, s1;
  if (!R.gather_range(t, s0, s1, tid)) return;
  const int L = s1 - s0, K = A.K;
  if (L <= K) return;
  const float* row = R.row(t) + s0;
  const int64_t lo = (int64_t)L * g / A.gsplit, hi = (int64_t)L * (g + 1) / A.gsplit;
  const int64_t region = ((int64_t)t * A.gsplit + g) * A.gcap;
  uint32_t* gk = A.gkey + region;
  int32_t* gi = A.gid + region;
  constexpr int U = 16;
  constexpr int kStep = kWG * U;
  constexpr int kRounds = 4;  // slices up to kRounds * kStep keys stay in registers
  // the sample's loads first, then the whole slice's (clamped, no branch),
  // so that the slice arrives while the cut is being selected; R rounds of
  // U loads per thread, R the fewest that cover the slice
  const auto in_regs = [&](auto RC) {
    constexpr int R = decltype(RC)::value;
    uint32_t sk[kSampleBlocks];
    sample_load(row, L, sk, tid);
    uint32_t k[R][U];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) k[r][u] = f2key(row[min(lo + r * kStep + u * kWG + tid, hi - 1)]);
    const uint32_t cut = sample_select(sk, L, K, sh, tid);
    uint32_t cnt = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) cnt += ((lo + r * kStep + u * kWG + tid < hi) & (k[r][u] >= cut)) ? 1u : 0u;
    uint32_t total;
    uint32_t slot = block_exclusive_scan(cnt, sh, tid, total);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = lo + r * kStep + u * kWG + tid;
        if ((i < hi) & (k[r][u] >= cut)) {
          if (slot < (uint32_t)A.gcap) {
            gk[slot] = k[r][u];
            gi[slot] = (int32_t)i + s0;
          }
          ++slot;
        }
      }
    if (tid == 0) A.gcnt[(int64_t)t * A.gsplit + g] = total;
  };
  const int64_t n = hi - lo;
  if (n <= kStep) return in_regs(std::integral_constant<int, 1>{});
  if (n <= 2 * kStep) return in_regs(std::integral_constant<int, 2>{});
  if (n <= kRounds * kStep) return in_regs(std::integral_constant<int, kRounds>{});
  const uint32_t cut = sample_cut(row, L, K, sh, tid);
  // longer slices, pass 1: per-thread counts, U loads in flight and no barrier; one
  // workgroup scan gives each thread its first slot; pass 2 re-reads the
  // slice (from L2) in threads that found keys and writes them.  A scan per
  // round of loads would wait out a memory latency per round.  Loads past
  // the slice read its last element (clamped index, not a branch: a load
  // behind a branch is waited for at once) and are not counted.
  uint32_t cnt = 0u;
#pragma unroll 1
  for (int64_t base = lo; base < hi; base += kStep) {
    uint32_t k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) k[u] = f2key(row[min(base + u * kWG + tid, hi - 1)]);
#pragma unroll
    for (int u = 0; u < U; ++u) cnt += ((base + u * kWG + tid < hi) & (k[u] >= cut)) ? 1u : 0u;
  }
  uint32_t total;
  uint32_t slot = block_exclusive_scan(cnt, sh, tid, total);
  if (cnt != 0u && slot < (uint32_t)A.gcap) {
#pragma unroll 1
    for (int64_t base = lo; base < hi; base += kStep) {
      uint32_t k[U];
#pragma unroll
      for (int u = 0; u < U; ++u) k[u] = f2key(row[min(base + u * kWG + tid, hi - 1)]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + u * kWG + tid;
        if ((i < hi) & (k[u] >= cut)) {
          if (slot < (uint32_t)A.gcap) {
            gk[slot] = k[u];
            gi[slot] = (int32_t)i + s0;
          }
          ++slot;
        }
      }
    }
  }
  if (tid == 0) A.gcnt[(int64_t)t * A.gsplit + g] = total;
}

int launch_topk_rows_gathered(const RowsArgs& A, hipStream_t stream) {
  if (A.Q == 0) return IDX_OK;
  if (!A.gkey || A.gsplit < 1 || A.gsplit > kMaxGatherSplit || (A.gsplit & (A.gsplit - 1)) || A.gcap < 1 ||
      A.gcap * A.gsplit > kRowsCap)
    return IDX_EINVAL;
  if (A.Q > kMaxGridY) return IDX_EUNSUPPORTED;  // rows index the gather grid's y dimension
  if (A.table) {
    hipLaunchKernelGGL(k_rows_gather<PagedRows>, dim3(A.gsplit, A.Q), dim3(kWG), 0, stream, A);
    hipLaunchKernelGGL((k_topk_rows<PagedRows, kMaxWaves>), dim3(A.Q), dim3(64 * kMaxWaves), 0, stream, A);
  } else {
    hipLaunchKernelGGL(k_rows_gather<DenseRows>, dim3(A.gsplit, A.Q), dim3(kWG), 0, stream, A);
    hipLaunchKernelGGL((k_topk_rows<DenseRows, kWaves>), dim3(A.Q), dim3(kWG), 0, stream, A);
  }
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

int launch_topk_rows_filtered(const RowsArgs& A, hipStream_t stream) {
  if (A.Q == 0) return IDX_OK;
  if (!A.table || !A.dcnt || !A.dcand || !A.dplan || A.dseg < 1 || A.gcnt) return IDX_EINVAL;
  hipLaunchKernelGGL((k_topk_rows<PagedRows, kMaxWaves>), dim3(A.Q), dim3(64 * kMaxWaves), 0, stream, A);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

int launch_topk_rows(const RowsArgs& A, hipStream_t stream) {
  if (A.Q == 0) return IDX_OK;
  if (A.table) return IDX_EINVAL;  // paged rows go through the filtered or pre-gathered launches
  hipLaunchKernelGGL((k_topk_rows<DenseRows, kWaves>), dim3(A.Q), dim3(kWG), 0, stream, A);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

}  // namespace idxk
