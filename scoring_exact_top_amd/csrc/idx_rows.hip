// Exact top-K over a dense FP32 score matrix, one workgroup per row: the
// standalone selection stage of an unfused pipeline (Fusing Indexer Scoring
// and Exact Top-k page, "2.1 Where the cost goes" and Table 2: score into an
// explicit [Q,N] matrix, then select), kept as the comparator for the fused
// path and as a library routine of its own.
//
// Per row of length L > K:
//   0. a cut c from a sample of the row: kSampleBlocks contiguous blocks of
//      256 scores spread over it, c = a sample key with about 2K of the
//      row's keys expected at or above it (the page's sampled threshold,
//      "3.2 Sampled threshold", applied to an explicit score row);
//   1. one streaming pass gathers every key >= c into LDS; with K to
//      kRowsCap of them, the register-resident range select over the
//      gathered keys finishes the row (ties at the K-th score to the lowest
//      ids): one read of the row in all.
// Otherwise (a short row without a sample, or a cut that kept too few or
// too many keys) two more passes: a 2048-bin histogram of the top 11 bits
// of the order-preserving keys (>= c when c kept too many) finds the bin b
// of the K-th largest key ("3.2": radix select on order-preserving 32-bit
// integers); the next pass writes out every key in a bin above b and
// gathers bin b, which the range select finishes.  A bin too large for LDS
// (massive ties) goes to the generic four-digit radix select over the row
// in memory, with the same tie rule.
#include "idx_internal.hpp"
#include "idx_rows.hpp"

namespace idxk {

constexpr int kRowsBins = 2048;
constexpr int kRowsShift = 21;  // 32 - 11 bits
constexpr int kRowsCap = 6144;  // gathered keys held in LDS
constexpr int kRowsRegs = kRowsCap / kWG;
constexpr int kRowsUnroll = 4;  // 16-byte loads per thread per pass step (two steps in flight)
constexpr int kSampleBlocks = 16;  // sample: 16 blocks of kWG scores
constexpr int kSampleKeys = kSampleBlocks * kWG;
constexpr int kSampleMinLen = 4 * kSampleKeys;  // shorter rows are not sampled

// Dense row in memory: element i is position s0 + i.
struct SrcDense {
  const float* row;
  int32_t s0;
  __device__ uint32_t key(int i) const { return f2key(row[i]); }
  __device__ int32_t id(int i) const { return s0 + i; }
};

// Calls f(i, valid, key) for every element i < L of the row (and for some
// positions outside it with valid = false), reading it with 16-byte buffer
// loads from the 16-byte-aligned address at or below the row's start (reads
// past the end return 0); the next step's loads are issued before this
// step's keys are processed.
template <class F>
__device__ __forceinline__ void for_each_key(const float* row, int L, int tid, const F& f) {
  const int shift = (int)(((uintptr_t)row & 15u) >> 2);  // elements before the row in its first 16 bytes
  const float* abase = row - shift;
  const int span = L + shift;
  const rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, span * 4, 0x00020000);
  constexpr int kStep = kWG * 4 * kRowsUnroll;
  const auto load = [&](v4i (&v)[kRowsUnroll], int base) {
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rr, (base + (u * kWG + tid) * 4) * 4, 0, 0);
  };
  v4i cur[kRowsUnroll];
  load(cur, 0);
  for (int base = 0; base < span; base += kStep) {
    v4i nxt[kRowsUnroll];
    load(nxt, base + kStep);
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
      const int i0 = base + (u * kWG + tid) * 4 - shift;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        f(i, i >= 0 && i < L, f2key(__int_as_float(cur[u][e])));
      }
    }
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) cur[u] = nxt[u];
  }
}

struct RowsShared {
  union {
    uint32_t hist[kRowsBins];  // histogram path, before the gather
    uint32_t lkey[kRowsCap];
  };
  int32_t lid[kRowsCap];
  uint32_t n_gt, n_eq, bin, above, inbin, pad[3];
  SelShared sh;
};

// Exact selection of the rem largest of the n gathered keys (ties to the
// lowest ids), written to out[0, rem).  1 <= rem <= n <= kRowsCap.  All
// threads call this.
__device__ void select_gathered(RowsShared& S, uint32_t n, int rem, int32_t* out, int tid) {
  const RegLayout lay = block_list_layout(n, (uint32_t)tid);
  uint32_t key[kRowsRegs];
  int32_t id[kRowsRegs];
#pragma unroll
  for (int j = 0; j < kRowsRegs; ++j) {
    const bool v = lay.valid(j);
    key[j] = v ? S.lkey[lay.at(j)] : 0u;
    id[j] = v ? S.lid[lay.at(j)] : 0;
  }
  const auto kf = [&](int j) { return key[j]; };
  const RangeSel sel = (n > (uint32_t)rem) ? range_select_regs<kRowsRegs>(kf, lay, rem, S.sh, tid)
                                            : RangeSel{1u, 0xFFFFFFFFu, rem, (int)n};
  const uint32_t idlo = tie_bound_regs(key, id, lay, sel, S.sh, tid);
  emit_range_regs(key, id, lay, sel, idlo, rem, rem, out, IdIdentity{}, S.sh, tid);
}

__global__ __launch_bounds__(kWG, 3) void k_topk_rows(RowsArgs A) {
  __shared__ RowsShared S;
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  int32_t* out = A.out + (int64_t)t * A.K;
  uint32_t* stats = A.ctrl ? stat_copy(A.ctrl, blockIdx.x) : nullptr;
  if (stats && tid == 0) atomicAdd(&stats[kStRows], 1u);
  const int s0 = A.row_start[t], s1 = A.row_end[t];
  if (s0 < 0 || s0 > s1 || s1 > A.N) {
    for (int i = tid; i < A.K; i += kWG) out[i] = -1;
    if (stats && tid == 0) atomicAdd(&stats[kStBad], 1u);
    return;
  }
  const int L = s1 - s0;
  const int K = A.K;
  if (L <= K) {  // every key of the row, in position order
    for (int i = tid; i < K; i += kWG) out[i] = i < L ? s0 + i : -1;
    if (stats && tid == 0) atomicAdd(&stats[kStTrivial], 1u);
    return;
  }
  const float* row = A.scores + (int64_t)t * A.ld + s0;

  // step 0: the sampled cut (key 0 keeps every key)
  uint32_t cut = 0u;
  if (L >= kSampleMinLen) {
    uint32_t sk[kSampleBlocks];
    const int64_t span = (int64_t)L - kWG;
#pragma unroll
    for (int j = 0; j < kSampleBlocks; ++j)
      sk[j] = f2key(row[span * j / (kSampleBlocks - 1) + tid]);
    // rank r in the sample <=> about r * L / kSampleKeys keys of the row
    const int r = (int)(((int64_t)2 * K * kSampleKeys + L - 1) / L);
    if (r < kSampleKeys) {
      const RegLayout lay{(uint32_t)tid, (uint32_t)kWG, (uint32_t)kSampleKeys, (uint32_t)kSampleBlocks};
      cut = range_select_regs<kSampleBlocks>([&](int j) { return sk[j]; }, lay, r, S.sh, tid).lo;
    }
  }

  // step 1: one pass gathering the keys at or above the cut
  if (cut) {
    if (tid == 0) S.n_eq = 0u;
    __syncthreads();
    for_each_key(row, L, tid, [&](int i, bool v, uint32_t key) {
      const bool ge = v && key >= cut;
      if (__ballot(ge)) {
        const uint32_t pe = reserve(&S.n_eq, ge);
        if (ge && pe < (uint32_t)kRowsCap) { S.lkey[pe] = key; S.lid[pe] = s0 + i; }
      }
    });
    __syncthreads();
    const uint32_t n = S.n_eq;
    if (n >= (uint32_t)K && n <= (uint32_t)kRowsCap) {
      select_gathered(S, n, K, out, tid);
      if (stats && tid == 0) atomicAdd(&stats[kStFast], 1u);
      return;
    }
    if (n < (uint32_t)K) cut = 0u;  // the cut kept too few keys: histogram the whole row
    __syncthreads();
  }

  // histogram path: the bin of the K-th largest key among keys >= cut
  for (int i = tid; i < kRowsBins; i += kWG) S.hist[i] = 0u;
  if (tid == 0) { S.n_gt = 0u; S.n_eq = 0u; }
  __syncthreads();
  for_each_key(row, L, tid, [&](int, bool v, uint32_t key) {
    hist_add(S.hist, key >> kRowsShift, v && key >= cut);  // returns at once when no lane qualifies
  });
  __syncthreads();
  {
    // thread u holds bins 8u .. 8u+7
    uint32_t h[8], a = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) { h[j] = S.hist[8 * tid + j]; a += h[j]; }
    uint32_t total;
    const uint32_t before = block_exclusive_scan(a, S.sh, tid, total);
    uint32_t ab = total - before - a;  // keys in bins above this thread's
    const uint32_t r = (uint32_t)K;
    if (ab < r && r <= ab + a) {
#pragma unroll
      for (int j = 7; j >= 0; --j) {
        if (ab < r && r <= ab + h[j]) { S.bin = 8u * tid + j; S.above = ab; S.inbin = h[j]; }
        ab += h[j];
      }
    }
  }
  __syncthreads();
  const uint32_t bin = S.bin, above = S.above, inbin = S.inbin;

  // keys above the bin go straight out; the bin's keys (>= cut) to LDS
  for_each_key(row, L, tid, [&](int i, bool v, uint32_t key) {
    const uint32_t d = key >> kRowsShift;
    const bool gt = v && d > bin, eq = v && d == bin && key >= cut;
    if (__ballot(gt || eq)) {
      const uint32_t pg = reserve(&S.n_gt, gt);
      if (gt) out[pg] = s0 + i;
      const uint32_t pe = reserve(&S.n_eq, eq);
      if (eq && pe < (uint32_t)kRowsCap) { S.lkey[pe] = key; S.lid[pe] = s0 + i; }
    }
  });
  __syncthreads();

  const int rem = K - (int)above;  // 1 <= rem <= inbin
  if (inbin <= (uint32_t)kRowsCap) {
    select_gathered(S, inbin, rem, out + above, tid);
    if (stats && tid == 0) atomicAdd(&stats[kStFast], 1u);
  } else {
    // the bin does not fit: exact radix select over the row in memory
    const SrcDense src{row, s0};
    const SelResult sel = radix_select(src, L, K, S.sh, tid, false, true);
    emit_selection(src, L, sel, K, K, out, S.sh, tid);
    if (stats && tid == 0) atomicAdd(&stats[kStRepaired], 1u);
  }
}

int launch_topk_rows(const RowsArgs& A, hipStream_t stream) {
  if (A.Q == 0) return IDX_OK;
  hipLaunchKernelGGL(k_topk_rows, dim3(A.Q), dim3(kWG), 0, stream, A);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

}  // namespace idxk
