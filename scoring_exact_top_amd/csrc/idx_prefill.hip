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

// ----------------------------------------------------------------- relayout

// One 16-byte chunk per thread: tile j, block b, lane l of the relaid copy
// (layout described with relaid_src_offset).  Keys past N read as zero.
__global__ __launch_bounds__(kWG) void k_relayout_keys(PrefillArgs A) {
  const int64_t chunk = (int64_t)blockIdx.x * kWG + threadIdx.x;  // 512 chunks per tile
  const int tile = (int)(chunk >> 9), blk = (int)((chunk >> 6) & 7), l = (int)(chunk & 63);
  const int key = (tile << 6) + sub_off(blk >> 1) + (l & 15);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (key < A.N) v = *reinterpret_cast<const uint4*>(A.k + relaid_src_offset(tile, blk, l));
  reinterpret_cast<uint4*>(A.kt)[chunk] = v;
}

// ------------------------------------------------------------------ sampler

// One workgroup per row: score the sampled keys exactly as the main pass
// does, then take the r-th largest as tau.
__global__ __launch_bounds__(kWG) void k_prefill_tau(PrefillArgs A) {
  __shared__ uint32_t s_samp[kMaxSamples];
  __shared__ SelShared sh;
  __shared__ uint8_t s_qprep[kWaves][kUTerms * kD];
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
  prepare_q(qo, A.q, A.q_scale, A.w, t, lane, s_qprep[tid >> 6]);
  const KeyBuf kbuf = make_keybuf(A.k, A.k_scale, A.N);
  const float tau = sample_tau(qo, kbuf, TileContig{}, s0, sg, s_samp, sh, tid);
  if (tid == 0) A.tau[t] = tau;
}

// ------------------------------------------------------------- fused main

// Per-wave candidate bookkeeping of the main kernel.
struct CandState {
  uint32_t cnt;      // candidates seen (may exceed the capacity)
  uint32_t staged;   // entries in the LDS stage
  uint32_t flushed;  // entries already in the workspace list
};

// Copy the wave's LDS stage to its workspace list (as far as capacity
// allows) and empty it.  Rare: once per ~kStage candidates.
__device__ __forceinline__ void flush_stage(CandState& cs, uint2* stage, uint32_t* gk, int32_t* gi,
                                            uint32_t cap, uint32_t lane) {
  wave_sync();
  for (uint32_t i = lane; i < cs.staged; i += 64) {
    const uint32_t o = cs.flushed + i;
    if (o < cap) {
      const uint2 e = stage[i];
      gk[o] = e.x;
      gi[o] = (int32_t)e.y;
    }
  }
  cs.flushed = min(cs.flushed + cs.staged, cap);
  cs.staged = 0;
  wave_sync();
  // Drain the stores here (vmcnt(0), other counters untouched) so that the
  // common no-flush path never has to assume stores in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Epilogue phase for one tile: scores of keys key0..key0+63 (lane l: key0+l)
// from the accumulators, range mask, threshold filter and staging.
template <bool DBG>
__device__ __forceinline__ void main_epilogue(const QOp& qo, const v4f (&acc)[20], float ks, int key0,
                                              int rs, int re, float tau, float* dbg, CandState& cs,
                                              uint2* stage, uint32_t stage_cap, uint32_t* gk,
                                              int32_t* gi, uint32_t cap, uint32_t lane) {
  const int my = key0 + (int)lane;
  const float sc = tile_epilogue(qo, acc) * ks;
  const bool valid = my >= rs && my < re;
  if (DBG && valid) dbg[my] = sc;
  const bool take = valid && sc >= tau;
  const uint64_t ball = __ballot(take);
  if (ball) {
    const uint32_t n = (uint32_t)__popcll(ball);
    if (cs.staged + n > stage_cap) flush_stage(cs, stage, gk, gi, cap, lane);
    if (take) stage[cs.staged + rank_in(ball)] = make_uint2(f2key(sc), (uint32_t)my);
    cs.staged += n;
    cs.cnt += n;
  }
}

// Eight waves, one query row each, walk the same 64-key tiles of the rows'
// union range.  Waves w and w+4 share a SIMD and run in opposite phases:
// while one issues the 16 MFMAs of a tile, the other runs the VALU epilogue
// of its previous tile, so the matrix core and the vector ALU work at the same
// time.  Execution barriers swap the phases.  Key tiles are prefetched into
// registers two phases ahead; the epilogue touches only LDS.  After the walk
// every wave certifies and selects its own row.
// DBG: also write every valid score to A.dbg_scores (test/diagnosis build of
// the same arithmetic; the production instantiation has no store in its
// epilogue).
template <bool DBG>
__global__ __launch_bounds__(kMainThreads, 1) void k_prefill_main(PrefillArgs A) {
  __shared__ uint2 s_stage[kMainWaves][kStage];
  __shared__ uint32_t s_hist[kMainWaves][256];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int t0 = blockIdx.x * kMainWaves;
  const int t = t0 + wave;
  const bool row_ok = t < A.Q;
  const int tc = min(t, A.Q - 1);

  // union of the workgroup's valid ranges (every wave computes it alike)
  int lo = 0x7fffffff, hi = -1;
  for (int r = 0; r < kMainWaves && t0 + r < A.Q; ++r) {
    const int s = A.row_start[t0 + r], e = A.row_end[t0 + r];
    if (s >= 0 && s < e && e <= A.N) { lo = min(lo, s); hi = max(hi, e); }
  }
  int rs = 0, re = 0;
  bool bad = false;
  float tau = INFINITY;
  if (row_ok) {
    rs = A.row_start[t]; re = A.row_end[t];
    bad = rs < 0 || rs > re || re > A.N;
    if (bad) { rs = 0; re = 0; } else tau = A.tau[t];
  }
  QOp qo;
  prepare_q(qo, A.q, A.q_scale, A.w, tc, lane, reinterpret_cast<uint8_t*>(s_hist[wave]));
  const KeyBuf kbuf = make_keybuf(A.k, A.k_scale, A.N);

  const int tile_lo = lo >> 6;
  const int nt = lo < hi ? ((hi + 63) >> 6) - tile_lo : 0;
  const uint32_t cap = (uint32_t)min(A.cap_total, kCandCap);
  const uint32_t stage_cap = (uint32_t)max(64, min(A.lds_cap, kStage));
  uint2* stage = s_stage[wave];
  uint32_t* gk = A.cand_key + (int64_t)tc * kCandCap;
  int32_t* gi = A.cand_idx + (int64_t)tc * kCandCap;
  float* dbg = A.dbg_scores ? A.dbg_scores + (int64_t)tc * A.N : nullptr;
  CandState cs{0u, 0u, 0u};
  KeyTile b0, b1;
  v4f acc[20];

#define IDX_PHASE_BARRIER()            \
  do {                                 \
    __builtin_amdgcn_sched_barrier(0); \
    __builtin_amdgcn_s_barrier();      \
    __builtin_amdgcn_sched_barrier(0); \
  } while (0)
  // MFMA phase on tile j held in CUR, then prefetch tile j+1 into NXT.
#define IDX_M(j, CUR, NXT)                                                                     \
  do {                                                                                         \
    tile_mfma(qo, CUR.kb, acc);                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    /* unconditional: past the end the buffer reads return 0, and a fixed   \
       load count lets the epilogue wait only for the older loads it needs */ \
    load_tile(NXT, kbuf, (tile_lo + (j) + 1) << 6, lane);                                       \
  } while (0)
#define IDX_V(j, CUR)                                                                          \
  main_epilogue<DBG>(qo, acc, CUR.ks, (tile_lo + (j)) << 6, rs, re, tau, dbg, cs, stage, stage_cap, gk, gi, \
                cap, lane)

  if (nt > 0) load_tile(b0, kbuf, tile_lo << 6, lane);
  // One full drain before the loop: the loop's own wait analysis then only
  // sees its in-loop prefetches and waits for exactly the tile it needs.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // Each loop iteration handles two tiles with fixed register roles; an odd
  // last tile leaves through `break`, so the loop back-edge always carries
  // the same set of loads in flight.
  if (group == 0) {
    for (int j = 0; j < nt; j += 2) {
      IDX_M(j, b0, b1);
      IDX_PHASE_BARRIER();
      IDX_V(j, b0);
      IDX_PHASE_BARRIER();
      if (j + 1 >= nt) break;
      IDX_M(j + 1, b1, b0);
      IDX_PHASE_BARRIER();
      IDX_V(j + 1, b1);
      IDX_PHASE_BARRIER();
    }
  } else {
    int j = 0;
    if (nt > 0) {
      IDX_PHASE_BARRIER();
      IDX_M(0, b0, b1);
      IDX_PHASE_BARRIER();
      for (j = 1; j < nt; j += 2) {
        IDX_V(j - 1, b0);
        IDX_PHASE_BARRIER();
        IDX_M(j, b1, b0);
        IDX_PHASE_BARRIER();
        if (j + 1 >= nt) break;
        IDX_V(j, b1);
        IDX_PHASE_BARRIER();
        IDX_M(j + 1, b0, b1);
        IDX_PHASE_BARRIER();
      }
      // the last tile nt-1 sits in b0 when nt is odd, in b1 when even
      if (nt & 1) IDX_V(nt - 1, b0);
      else IDX_V(nt - 1, b1);
    }
  }
#undef IDX_V
#undef IDX_M
#undef IDX_PHASE_BARRIER

  // certificate + selection, one row per wave, no workgroup barrier
  if (!row_ok) return;
  wave_sync();
  uint32_t* stats = A.ctrl + kStatsOff;
  int32_t* out = A.out + (int64_t)t * A.K;
  if (lane == 0) atomicAdd(&stats[kStRows], 1u);
  if (bad) {
    for (int i = (int)lane; i < A.K; i += 64) out[i] = -1;
    if (lane == 0) atomicAdd(&stats[kStBad], 1u);
    return;
  }
  const int L = re - rs;
  const int kr = min(A.K, L);
  if (cs.cnt >= (uint32_t)kr && cs.cnt <= cap) {
    const SrcMain src{gk, gi, (int)cs.flushed, stage};
    const SelResult sel = (cs.cnt > (uint32_t)kr)
                              ? wave_radix_select(src, (int)cs.cnt, kr, s_hist[wave], lane, true)
                              : SelResult{0u, 0u, kr};
    wave_emit(src, (int)cs.cnt, sel, kr, A.K, out, lane);
    if (lane == 0) {
      atomicAdd(&stats[kStFast], 1u);
      if (cs.flushed > 0) atomicAdd(&stats[kStSpilled], 1u);
      if (L <= A.K) atomicAdd(&stats[kStTrivial], 1u);
    }
  } else if (lane == 0) {
    const uint32_t f = atomicAdd(&A.ctrl[kCtrlFail], 1u);
    A.fail_list[f] = t;
    atomicAdd(&stats[cs.cnt < (uint32_t)kr ? kStUnder : kStOver], 1u);
  }
}

// ------------------------------------------------------ paired-row main

// Two query rows per workgroup of four waves; two workgroups per CU.  Each
// wave walks every fourth 64-key tile of the rows' union range and, per
// 16-key sub-tile, issues the 9 MFMAs of both rows (4 head blocks each plus
// the shared u block), refills that sub-tile's registers with the same
// sub-tile of its next tile (a rolling prefetch one tile ahead), and folds
// the results into the rows' partial sums; the compiler interleaves the next
// MFMAs with this epilogue.  Keys >= tau are appended, as raw score bits
// and key id, to a per-(row, wave) LDS stage whose fill level is a scalar
// count (ballot + popcount, no atomics); a full stage is copied in bulk to
// the wave's private segment of the row's workspace candidate area.  After
// the walk the workgroup certifies and selects each row in turn, reading the
// row's four segments as one list.
template <bool DBG>
__global__ __launch_bounds__(kWG, 2) void k_prefill_pair(PrefillArgs A) {
  __shared__ uint2 s_stage[2][kWaves][kSegStage];
  __shared__ uint32_t s_segn[2][kWaves];   // entries in each segment (capped)
  __shared__ uint32_t s_segover[2];        // some segment of the row overflowed
  __shared__ SelShared sh;
  __shared__ uint8_t s_qprep[kWaves][2 * kUTerms * kD];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = 2 * blockIdx.x;

  int rs[2], re[2];
  float tr[2];
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
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
  if (tid < 2) s_segover[tid] = 0u;
  QOp2 qo;
  prepare_q2(qo, A.q, A.q_scale, A.w, min(t0, A.Q - 1), min(t0 + 1, A.Q - 1), lane, s_qprep[wave]);
  __syncthreads();

  const KeyBuf kbuf = make_keybuf(A.k, A.k_scale, A.N);
  const int ntiles = (A.N + 63) >> 6;
  const rsrc_t ktb = __builtin_amdgcn_make_buffer_rsrc((void*)A.kt, (short)0, ntiles * kTile * kD, 0x00020000);
  // per-segment capacities (the debug knobs scale them down)
  const uint32_t seg_cap = (uint32_t)min(kSegCap, A.cap_total / kWaves);
  const uint32_t stage_cap = (uint32_t)max(64, min(kSegStage, A.lds_cap / kWaves));
  const int tile_hi = (hi + 63) >> 6;
  const int voff = (int)lane * 16;
  uint32_t cnt[2] = {0u, 0u}, staged[2] = {0u, 0u}, flushed[2] = {0u, 0u};
  uint32_t* segk[2];
  int32_t* segi[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int64_t o = ((int64_t)min(t0 + r, A.Q - 1) * kWaves + wave) * kSegCap;
    segk[r] = A.cand_key + o;
    segi[r] = A.cand_idx + o;
  }
  // Copy row r's LDS stage to its workspace segment (as far as capacity
  // allows) and empty it; drain the stores so the loop's waits stay exact.
  auto flush = [&](int r) {
    wave_sync();
    for (uint32_t i = lane; i < staged[r]; i += 64) {
      const uint32_t o = flushed[r] + i;
      if (o < seg_cap) {
        const uint2 e = s_stage[r][wave][i];
        segk[r][o] = e.x;
        segi[r][o] = (int32_t)e.y;
      }
    }
    flushed[r] = min(flushed[r] + staged[r], seg_cap);
    staged[r] = 0u;
    wave_sync();
    __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  // One tile: 9 MFMAs per 16-key sub-tile on CUR (both rows' head blocks and
  // the shared u block), then that sub-tile's slice of tile T+4 is loaded
  // into NXT (the other buffer: a whole tile of lead, no register copies),
  // then the sub-tile's epilogue.  Reads past the end return 0.
  auto tile_body = [&](int T, const v8i (&cur)[4], v8i (&nxt)[4], float ks_cur, float& ks_nxt) {
    const int ntoff = (T + kWaves) * (kTile * kD);
    float p0[4], p1[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v4f a0[4], a1[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        a0[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[0][b], cur[c], z, 0, 0, 0, 0, 0, 0);
        a1[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[1][b], cur[c], z, 0, 0, 0, 0, 0, 0);
      }
      const v4f au = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.au, cur[c], z, 0, 0, 0, 0, 0, 0);
      nxt[c] = cat8(__builtin_amdgcn_raw_buffer_load_b128(ktb, voff, ntoff + (2 * c) * 1024, 0),
                    __builtin_amdgcn_raw_buffer_load_b128(ktb, voff, ntoff + (2 * c + 1) * 1024, 0));
      __builtin_amdgcn_sched_group_barrier(0x008, 9, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x0 = fmaf(qo.wh[0][4 * b + r], fabsf(a0[b][r]), x0);
          x1 = fmaf(qo.wh[1][4 * b + r], fabsf(a1[b][r]), x1);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x0 = fmaf(qo.sh[0][r], au[r], x0);
        x1 = fmaf(qo.sh[1][r], au[r], x1);
      }
      p0[c] = x0;
      p1[c] = x1;
      __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);
    }
    ks_nxt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kbuf.ks, (int)lane * 4, ntoff / kD * 4, 0));
    const float sc[2] = {reduce_scatter4(p0[0], p0[1], p0[2], p0[3]) * ks_cur,
                         reduce_scatter4(p1[0], p1[1], p1[2], p1[3]) * ks_cur};
    const int my = (T << 6) + (int)lane;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const bool valid = my >= rs[r] && my < re[r];
      if (DBG && valid) A.dbg_scores[(int64_t)(t0 + r) * A.N + my] = sc[r];
      const bool take = valid && sc[r] >= tr[r];
      const uint64_t ball = __ballot(take);
      if (ball) {
        const uint32_t n = (uint32_t)__popcll(ball);
        if (staged[r] + n > stage_cap) flush(r);
        if (take) s_stage[r][wave][staged[r] + rank_in(ball)] = make_uint2(__float_as_uint(sc[r]), (uint32_t)my);
        staged[r] += n;
        cnt[r] += n;
      }
    }
  };
  if (lo < hi) {
    int T = (lo >> 6) + wave;
    v8i kA[4], kB[4];
    float sA, sB;
    {
      KeyTile t;
      load_tile_relaid(t, ktb, kbuf.ks, T, lane);
#pragma unroll
      for (int c = 0; c < 4; ++c) kA[c] = t.kb[c];
      sA = t.ks;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // drain once so the loop's waits stay exact
    for (;;) {
      if (T >= tile_hi) break;
      tile_body(T, kA, kB, sA, sB);
      T += kWaves;
      if (T >= tile_hi) break;
      tile_body(T, kB, kA, sB, sA);
      T += kWaves;
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (staged[r]) flush(r);
    if (lane == 0) {
      s_segn[r][wave] = flushed[r];
      if (cnt[r] > seg_cap) s_segover[r] = 1u;
    }
  }
  __syncthreads();

  uint32_t* stats = A.ctrl + kStatsOff;
#pragma unroll 1
  for (int r = 0; r < 2; ++r) {
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
    const uint32_t n0 = s_segn[r][0], n1 = s_segn[r][1], n2 = s_segn[r][2], n3 = s_segn[r][3];
    const uint32_t n = n0 + n1 + n2 + n3;
    const bool complete = s_segover[r] == 0u;
    if (complete && n >= (uint32_t)kr) {
      const int64_t o = (int64_t)t * kWaves * kSegCap;
      const SrcSeg4 src{A.cand_key + o, A.cand_idx + o, (int)n0, (int)(n0 + n1), (int)(n0 + n1 + n2)};
      const SelResult sel = (n > (uint32_t)kr) ? radix_select(src, (int)n, kr, sh, tid, false, true)
                                              : SelResult{0u, 0u, kr};
      emit_selection(src, (int)n, sel, kr, A.K, out, sh, tid);
      if (tid == 0) {
        atomicAdd(&stats[kStFast], 1u);
        if (n > (uint32_t)(kWaves * min(kSegStage, max(64, A.lds_cap / kWaves)))) atomicAdd(&stats[kStSpilled], 1u);
        if (L <= A.K) atomicAdd(&stats[kStTrivial], 1u);
      }
    } else if (tid == 0) {
      const uint32_t f = atomicAdd(&A.ctrl[kCtrlFail], 1u);
      A.fail_list[f] = t;
      atomicAdd(&stats[complete ? kStUnder : kStOver], 1u);
    }
    __syncthreads();
  }
}

// ---------------------------------------------- 12-wave main (3 per SIMD)

constexpr int kTripRows = 4;    // query rows per workgroup
constexpr int kTripParts = 2;   // waves per row (interleaved tiles)
constexpr int kTripWaves = kTripRows * kTripParts;
constexpr int kTripThreads = 64 * kTripWaves;

// Twelve waves, three per SIMD: four query rows per workgroup, each row's
// tiles dealt round-robin to three waves.  One row per wave keeps the
// register footprint within a third of the SIMD's register file, so that
// while one wave issues MFMAs two others can issue epilogue VALU.  4096 rows
// fill 1024 workgroups = four full rounds of the 256 CUs.  Per 16-key
// sub-tile a wave issues the 5 MFMAs (4 head blocks + u block), refills
// those operand registers with the same sub-tile one tile ahead, then folds
// the results into the key's partial sum.  Candidates of a row go to its LDS
// area (then its spill area), slots reserved with one LDS atomic per wave;
// after the walk one wave per row selects it.
template <bool DBG>
__global__ __launch_bounds__(kTripThreads, 1) void k_prefill_trip(PrefillArgs A) {
  __shared__ uint32_t s_key[kTripRows][kLdsCap];
  __shared__ int32_t s_idx[kTripRows][kLdsCap];
  __shared__ uint32_t s_cnt[kTripRows];
  __shared__ uint8_t s_qprep[kTripWaves][kUTerms * kD];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = wave / kTripParts, part = wave % kTripParts;
  const int t0 = blockIdx.x * kTripRows;
  const int t = t0 + row;
  const bool row_ok = t < A.Q;

  int lo = 0x7fffffff, hi = -1;
  for (int r = 0; r < kTripRows && t0 + r < A.Q; ++r) {
    const int s = A.row_start[t0 + r], e = A.row_end[t0 + r];
    if (s >= 0 && s < e && e <= A.N) { lo = min(lo, s); hi = max(hi, e); }
  }
  int rs = 0, re = 0;
  float tau = INFINITY;
  if (row_ok) {
    const int s = A.row_start[t], e = A.row_end[t];
    if (s >= 0 && s <= e && e <= A.N) { rs = s; re = e; tau = A.tau[t]; }
  }
  if (tid < kTripRows) s_cnt[tid] = 0u;
  QOp qo;
  prepare_q(qo, A.q, A.q_scale, A.w, min(t, A.Q - 1), lane, s_qprep[wave]);
  __syncthreads();

  const KeyBuf kbuf = make_keybuf(A.k, A.k_scale, A.N);
  const uint32_t lcap = (uint32_t)A.lds_cap, scap = (uint32_t)A.spill_cap;
  const int tile_hi = (hi + 63) >> 6;
  const int voff = (int)(lane & 15) * kD + 32 * (int)(lane >> 4);
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  if (lo < hi) {
    int T = (lo >> 6) + part;
    v8i kb[4];
    float ks_cur, ks_nxt;
    {
      KeyTile kt;
      load_tile(kt, kbuf, T << 6, lane);
#pragma unroll
      for (int c = 0; c < 4; ++c) kb[c] = kt.kb[c];
      ks_cur = kt.ks;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // drain once so the loop's waits stay exact
    // Software pipeline over 16-key sub-tiles: stage c issues the MFMAs of
    // the next sub-tile (one by one, between the VALU ops of this sub-tile's
    // epilogue) into the other accumulator set, then refills that sub-tile's
    // operand registers one tile ahead.  issue(c) always writes acc[c & 1].
    v4f acc[2][5];
    auto issue = [&](v4f (&a)[5], const v8i& b) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        a[h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[h], b, z, 0, 0, 0, 0, 0, 0);
      a[4] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.au, b, z, 0, 0, 0, 0, 0, 0);
    };
    auto refill = [&](v8i& b, int base_key, int c) {
      const int soff = (base_key + sub_off(c)) * kD;
      b = cat8(__builtin_amdgcn_raw_buffer_load_b128(kbuf.k, voff, soff, 0),
               __builtin_amdgcn_raw_buffer_load_b128(kbuf.k, voff + 16, soff, 0));
    };
    auto epi = [&](const v4f (&a)[5]) {
      float x = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) x = fmaf(qo.wh[4 * h + r], fabsf(a[h][r]), x);
#pragma unroll
      for (int r = 0; r < 4; ++r) x = fmaf(qo.sh[r], a[4][r], x);
      return x;
    };
    issue(acc[0], kb[0]);
    refill(kb[0], (T + kTripParts) << 6, 0);
    for (;;) {
      const int nbase = (T + kTripParts) << 6;  // this wave's next tile (reads past the end return 0)
      const bool more = T + kTripParts < tile_hi;
      float p[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c < 3) {
          issue(acc[(c + 1) & 1], kb[c + 1]);
        } else if (more) {
          issue(acc[0], kb[0]);
        }
        p[c] = epi(acc[c & 1]);
        // interleave: one MFMA then four epilogue VALU ops, five times
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        if (c < 3) {
          refill(kb[c + 1], nbase, c + 1);
          if (c == 0)
            ks_nxt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kbuf.ks, (int)lane * 4, nbase * 4, 0));
        } else {
          refill(kb[0], nbase + (kTripParts << 6), 0);
        }
      }
      const float sc = reduce_scatter4(p[0], p[1], p[2], p[3]) * ks_cur;
      ks_cur = ks_nxt;
      const int my = (T << 6) + (int)lane;
      const bool valid = my >= rs && my < re;
      if (DBG && valid) A.dbg_scores[(int64_t)t * A.N + my] = sc;
      const bool take = valid && sc >= tau;
      const uint32_t pos = reserve(&s_cnt[row], take);
      if (take) {
        const uint32_t key = f2key(sc);
        if (pos < lcap) {
          s_key[row][pos] = key;
          s_idx[row][pos] = my;
        } else if (pos - lcap < scap) {
          const int64_t o = (int64_t)t * kCandCap + (pos - lcap);
          A.cand_key[o] = key;
          A.cand_idx[o] = my;
          __builtin_amdgcn_s_waitcnt(0x0F70);  // rare: keep the common path's waits exact
        }
      }
      if (!more) break;
      T += kTripParts;
    }
  }
  __syncthreads();
  if (!row_ok || part != 0) return;

  // one wave per row: certificate and selection
  uint32_t* stats = A.ctrl + kStatsOff;
  int32_t* out = A.out + (int64_t)t * A.K;
  if (lane == 0) atomicAdd(&stats[kStRows], 1u);
  const int rs_t = A.row_start[t], re_t = A.row_end[t];
  if (rs_t < 0 || rs_t > re_t || re_t > A.N) {
    for (int i = (int)lane; i < A.K; i += 64) out[i] = -1;
    if (lane == 0) atomicAdd(&stats[kStBad], 1u);
    return;
  }
  const int L = re_t - rs_t;
  const int kr = min(A.K, L);
  const uint32_t n = s_cnt[row];
  if (n >= (uint32_t)kr && n <= lcap + scap) {
    const SrcLdsSpill src{s_key[row], s_idx[row], (int)min(n, lcap), A.cand_key + (int64_t)t * kCandCap,
                          A.cand_idx + (int64_t)t * kCandCap};
    // the wave's 1 KiB of prepare scratch is free now: use it as the histogram
    uint32_t* hist = reinterpret_cast<uint32_t*>(s_qprep[wave]);
    const SelResult sel = (n > (uint32_t)kr) ? wave_radix_select(src, (int)n, kr, hist, lane, true)
                                            : SelResult{0u, 0u, kr};
    wave_emit(src, (int)n, sel, kr, A.K, out, lane);
    if (lane == 0) {
      atomicAdd(&stats[kStFast], 1u);
      if (n > lcap) atomicAdd(&stats[kStSpilled], 1u);
      if (L <= A.K) atomicAdd(&stats[kStTrivial], 1u);
    }
  } else if (lane == 0) {
    const uint32_t f = atomicAdd(&A.ctrl[kCtrlFail], 1u);
    A.fail_list[f] = t;
    atomicAdd(&stats[n < (uint32_t)kr ? kStUnder : kStOver], 1u);
  }
}

// ------------------------------------------------------------------ repair

// Exact repair of rows the certificate rejected: rescore the whole row into
// this workgroup's scratch slice as order-preserving keys, building the
// top-byte histogram on the way, then finish the radix select over the
// scratch.  Persistent: workgroup g handles failures g, g+G, ...
__global__ __launch_bounds__(kWG) void k_prefill_repair(PrefillArgs A) {
  __shared__ SelShared sh;
  __shared__ uint8_t s_qprep[kWaves][kUTerms * kD];
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
    prepare_q(qo, A.q, A.q_scale, A.w, t, lane, s_qprep[tid >> 6]);
    repair_row(qo, make_keybuf(A.k, A.k_scale, A.N), TileContig{}, IdIdentity{}, s0, s1, A.K,
               A.out + (int64_t)t * A.K, scratch, sh, tid);
    if (tid == 0) atomicAdd(&stats[kStRepaired], 1u);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ launch

int launch_prefill(const PrefillArgs& A, hipStream_t stream) {
  if (A.Q == 0) return IDX_OK;
  const int64_t nchunks = (int64_t)((A.N + 63) >> 6) * 512;
  if (nchunks > 0) hipLaunchKernelGGL(k_relayout_keys, dim3((unsigned)(nchunks / kWG)), dim3(kWG), 0, stream, A);
  hipLaunchKernelGGL(k_prefill_tau, dim3(A.Q), dim3(kWG), 0, stream, A);
  if (A.ev_main_start && hipEventRecord(A.ev_main_start, stream) != hipSuccess) return IDX_EHIP;
  if (A.dbg_scores)
    hipLaunchKernelGGL(k_prefill_pair<true>, dim3((A.Q + 1) / 2), dim3(kWG), 0, stream, A);
  else
    hipLaunchKernelGGL(k_prefill_pair<false>, dim3((A.Q + 1) / 2), dim3(kWG), 0, stream, A);
  if (A.ev_main_stop && hipEventRecord(A.ev_main_stop, stream) != hipSuccess) return IDX_EHIP;
  hipLaunchKernelGGL(k_prefill_repair, dim3(repair_grid(A.Q)), dim3(kWG), 0, stream, A);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

}  // namespace idxk
