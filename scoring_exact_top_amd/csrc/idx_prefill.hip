// Prefill path: sampled threshold -> fused score/filter/select -> exact repair.
//
// Fused Indexer Top-k page, "3.2 Sampled threshold: turn maintenance into
// filtering": each row gets a threshold tau from a sparse sample of its keys;
// the main pass keeps every key with score >= tau as a candidate (compare and
// append only), then an exact radix select over the candidates finds the
// K-th largest score.  Certificate: if all candidates were stored and there
// are at least K of them, the top-K of the candidates is the top-K of the row.
// Otherwise the row goes to the repair kernel, which rescores it into the
// workspace and selects exactly there.
#include "idx_common.hpp"
#include "idx_internal.hpp"

namespace idxk {

// ------------------------------------------------------------------ sampler

// One workgroup per row: score the sampled keys exactly as the main pass
// does, then take the r-th largest as tau.
__global__ __launch_bounds__(kWG) void k_prefill_tau(PrefillArgs A) {
  __shared__ uint32_t s_samp[kMaxSamples];
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  if (blockIdx.x == 0 && tid < kCtrlWords) A.ctrl[tid] = 0u;
  const int t = blockIdx.x;
  const int s0 = A.row_start[t], s1 = A.row_end[t];
  if (s0 < 0 || s0 > s1 || s1 > A.N) {
    if (tid == 0) A.tau[t] = INFINITY;
    return;
  }
  const int L = s1 - s0;
  if (A.force_tau) {
    if (tid == 0) A.tau[t] = A.tau_value;
    return;
  }
  const SampleGeom sg = sample_geom(L, A.cap_total);
  if (sg.n == 0) {
    if (tid == 0) A.tau[t] = -INFINITY;
    return;
  }
  QOp qo;
  load_q(qo, A.q, A.q_scale, A.w, t, lane);
  const float tau = sample_tau(qo, A.k, A.k_scale, MapIdentity{}, s0, sg, s_samp, sh, tid);
  if (tid == 0) A.tau[t] = tau;
}

// ------------------------------------------------------------- fused main

// BQ query rows per workgroup share every key load: the four waves walk the
// union of the rows' ranges in 64-key tiles, score each tile for all BQ rows
// from registers, and append (key32, id) of passing keys to the row's LDS
// candidate area (overflow goes to the row's spill area in the workspace).
// After the walk the workgroup runs the certificate and the radix select per
// row and writes the ids.
template <int BQ>
__global__ __launch_bounds__(kWG, 2) void k_prefill_fused(PrefillArgs A) {
  __shared__ uint32_t s_key[BQ][kLdsCap];
  __shared__ int32_t s_idx[BQ][kLdsCap];
  __shared__ uint32_t s_cnt[BQ];
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * BQ;

  int rs[BQ], re[BQ];
  float tr[BQ];
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int r = 0; r < BQ; ++r) {
    rs[r] = 0; re[r] = 0; tr[r] = INFINITY;
    const int t = t0 + r;
    if (t < A.Q) {
      const int s = A.row_start[t], e = A.row_end[t];
      if (s >= 0 && s <= e && e <= A.N) {
        rs[r] = s; re[r] = e; tr[r] = A.tau[t];
        if (e > s) { lo = min(lo, s); hi = max(hi, e); }
      }
    }
  }
  if (tid < BQ) s_cnt[tid] = 0u;
  QOp qo[BQ];
#pragma unroll
  for (int r = 0; r < BQ; ++r) load_q(qo[r], A.q, A.q_scale, A.w, min(t0 + r, A.Q - 1), lane);
  __syncthreads();

  const uint32_t lcap = (uint32_t)A.lds_cap, scap = (uint32_t)A.spill_cap;
  if (lo < hi) {
    const int tile_lo = lo >> 6, tile_hi = (hi + 63) >> 6;
    for (int tile = tile_lo + wave; tile < tile_hi; tile += kWaves) {
      const int key0 = tile << 6;
      const int my = key0 + (int)lane;
      float sc_all[BQ];
      score_tile<BQ>(qo, A.k, A.k_scale, MapIdentity{}, key0, lo, hi, lane, sc_all);
#pragma unroll
      for (int r = 0; r < BQ; ++r) {
        const float sc = sc_all[r];
        const bool valid = my >= rs[r] && my < re[r];
        if (A.dbg_scores && valid) A.dbg_scores[(int64_t)(t0 + r) * A.N + my] = sc;
        const bool take = valid && sc >= tr[r];
        const uint32_t pos = reserve(&s_cnt[r], take);
        if (take) {
          const uint32_t key = f2key(sc);
          if (pos < lcap) {
            s_key[r][pos] = key;
            s_idx[r][pos] = my;
          } else if (pos - lcap < scap) {
            const int64_t o = (int64_t)(t0 + r) * scap + (pos - lcap);
            A.spill_key[o] = key;
            A.spill_idx[o] = my;
          }
        }
      }
    }
  }
  __syncthreads();

  uint32_t* stats = A.ctrl + kStatsOff;
#pragma unroll 1
  for (int r = 0; r < BQ; ++r) {
    const int t = t0 + r;
    if (t >= A.Q) break;
    int32_t* out = A.out + (int64_t)t * A.K;
    if (tid == 0) atomicAdd(&stats[kStRows], 1u);
    const int rs_t = A.row_start[t], re_t = A.row_end[t];
    if (rs_t < 0 || rs_t > re_t || re_t > A.N) {
      for (int i = tid; i < A.K; i += kWG) out[i] = -1;
      if (tid == 0) atomicAdd(&stats[kStBad], 1u);
      continue;
    }
    const int L = re_t - rs_t;
    const int kr = min(A.K, L);
    const uint32_t n = s_cnt[r];
    if (n >= (uint32_t)kr && n <= lcap + scap) {
      const SrcLdsSpill src{s_key[r], s_idx[r], (int)min(n, lcap),
                            A.spill_key + (int64_t)t * scap, A.spill_idx + (int64_t)t * scap};
      const SelResult sel = (n > (uint32_t)kr) ? radix_select(src, (int)n, kr, sh, tid, false, true)
                                              : SelResult{0u, 0u, kr};
      emit_selection(src, (int)n, sel, kr, A.K, out, sh, tid);
      if (tid == 0) {
        atomicAdd(&stats[kStFast], 1u);
        if (n > lcap) atomicAdd(&stats[kStSpilled], 1u);
        if (L <= A.K) atomicAdd(&stats[kStTrivial], 1u);
      }
    } else if (tid == 0) {
      const uint32_t f = atomicAdd(&A.ctrl[kCtrlFail], 1u);
      A.fail_list[f] = t;
      atomicAdd(&stats[n < (uint32_t)kr ? kStUnder : kStOver], 1u);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ repair

// Exact repair of rows the certificate rejected: rescore the whole row into
// this workgroup's scratch slice as order-preserving keys, building the
// top-byte histogram on the way, then finish the radix select over the
// scratch.  Persistent: workgroup g handles failures g, g+G, ...
__global__ __launch_bounds__(kWG) void k_prefill_repair(PrefillArgs A) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t n_fail = __atomic_load_n(&A.ctrl[kCtrlFail], __ATOMIC_RELAXED);
  uint32_t* scratch = A.scratch + (int64_t)blockIdx.x * A.N;
  uint32_t* stats = A.ctrl + kStatsOff;
#pragma unroll 1
  for (uint32_t f = blockIdx.x; f < n_fail; f += gridDim.x) {
    const int t = A.fail_list[f];
    const int s0 = A.row_start[t], s1 = A.row_end[t];
    QOp qo;
    load_q(qo, A.q, A.q_scale, A.w, t, lane);
    repair_row(qo, A.k, A.k_scale, MapIdentity{}, IdIdentity{}, s0, s1, A.K, A.out + (int64_t)t * A.K,
               scratch, sh, tid);
    if (tid == 0) atomicAdd(&stats[kStRepaired], 1u);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ launch

int launch_prefill(const PrefillArgs& A, hipStream_t stream) {
  if (A.Q == 0) return IDX_OK;
  hipLaunchKernelGGL(k_prefill_tau, dim3(A.Q), dim3(kWG), 0, stream, A);
  if (A.ev_main_start && hipEventRecord(A.ev_main_start, stream) != hipSuccess) return IDX_EHIP;
  hipLaunchKernelGGL(k_prefill_fused<kBQ>, dim3((A.Q + kBQ - 1) / kBQ), dim3(kWG), 0, stream, A);
  if (A.ev_main_stop && hipEventRecord(A.ev_main_stop, stream) != hipSuccess) return IDX_EHIP;
  hipLaunchKernelGGL(k_prefill_repair, dim3(repair_grid(A.Q)), dim3(kWG), 0, stream, A);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

}  // namespace idxk
