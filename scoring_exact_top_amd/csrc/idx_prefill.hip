// Prefill path: sampled threshold -> fused score/filter/select -> exact repair.
//
// Fusing Indexer Scoring and Exact Top-k page, "3.2 Sampled threshold: turn maintenance into
// filtering": each row gets a threshold tau from a sparse sample of its keys;
// the main pass keeps every key with score >= tau as a candidate (compare and
// append only), then an exact radix select over the candidates finds the
// K-th largest score.  Certificate: if all candidates were stored and there
// are at least K of them, the top-K of the candidates is the top-K of the row.
// Otherwise the row goes to the repair kernel, which rescores it into the
// workspace and selects exactly there.
#include <hip/hip_ext.h>

#include "idx_common.hpp"
#include "idx_internal.hpp"
#include "idx_rows.hpp"

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
  if (A.keep_all || A.fuse_tau) {  // the sampler kernel is not launched: its other duties here
    if (blockIdx.x == 0) clear_ctrl(A.ctrl, threadIdx.x);
    const int64_t stride = (int64_t)gridDim.x * kWG;
    if (A.keep_all) {
      for (int64_t t = chunk; t < A.Q; t += stride) {
        const int s = A.row_start[t], e = A.row_end[t];
        A.tau[t] = (s >= 0 && s <= e && e <= A.N) ? -INFINITY : INFINITY;
      }
    } else {  // the main kernel writes the thresholds; the repair state starts at zero
      for (int64_t i = chunk; i < (int64_t)A.rslots * kRepairDigits * 256; i += stride) A.rhist[i] = 0u;
      for (int64_t i = chunk; i < (int64_t)A.rslots * kRowWords; i += stride) A.rrow[i] = 0u;
    }
  }
}

// ------------------------------------------------------------ thresholds

// Calls whose thresholds are not sampled by the main kernel (a forced
// threshold, which the unfused comparator and the test knobs use; or no
// keys at all): one thread per row sets tau (the forced value, +inf for an
// invalid range, -inf for an empty one); workgroup 0 clears the counters,
// and the repair state starts at zero.
__global__ __launch_bounds__(kWG) void k_prefill_tau(PrefillArgs A) {
  const int64_t i0 = (int64_t)blockIdx.x * kWG + threadIdx.x, stride = (int64_t)gridDim.x * kWG;
  if (blockIdx.x == 0) clear_ctrl(A.ctrl, threadIdx.x);
  for (int64_t i = i0; i < (int64_t)A.rslots * kRepairDigits * 256; i += stride) A.rhist[i] = 0u;
  for (int64_t i = i0; i < (int64_t)A.rslots * kRowWords; i += stride) A.rrow[i] = 0u;
  for (int64_t t = i0; t < A.Q; t += stride) {
    const int s = A.row_start[t], e = A.row_end[t];
    A.tau[t] = !(s >= 0 && s <= e && e <= A.N) ? INFINITY : A.force_tau ? A.tau_value : -INFINITY;
  }
}

// ------------------------------------------------------ paired-row main

// Every wave scores one pair of query rows; two workgroups of four waves per
// CU.  Two walks (prefill_geom):
//  - one-pair walk (SH = false): the four waves of a workgroup share one
//    pair, whose tiles are split over S workgroups (S*kWaves waves in all);
//    each wave walks every (S*kWaves)-th 64-key tile of the rows' union
//    range and refills each sub-tile's B operand straight from memory with
//    the same sub-tile of its next tile (one tile of lead);
//  - shared walk (SH = true): the four waves own four pairs (eight rows),
//    and all of them walk every S-th tile of the eight rows' union range;
//    each tile is staged once into LDS for all four waves (see
//    tile_body_shared).
// Per 16-key sub-tile a wave issues the 9 MFMAs of its pair (4 head blocks
// per row plus the shared u block), software-pipelined by row so that each
// row's epilogue runs under the other row's MFMAs.  Keys >= tau are stored,
// as raw score bits and key id, straight into the wave's private segment of
// the row's workspace candidate area; the slot comes from a scalar count
// plus the lane's rank in the ballot, so no atomics are involved.  After
// the walk each wave publishes its segment records; certification and
// selection follow in their own kernel.
//
// MODE kPairFused is that fused pass; kPairDebug also writes every valid
// score to dbg_scores [Q][N]; kPairDense only writes the scores (no filter,
// no candidates): the scoring stage of the unfused comparator.  kPairControl
// is the control of "5.2 Math-only control" (Fusing Indexer
// Scoring and Exact Top-k page): the same loads, MFMAs and scores, folded
// into one checksum per (row, segment) instead of being sampled, filtered and
// appended; with no selection or repair after it, the complete operator's
// time minus this kernel's is the selection work left exposed.
// kPairRepair rescores the rows the certificate rejected (exact repair,
// "3.2 Sampled threshold"): workgroups take the failure list's slotted
// rows two at a time, split each pair's tiles over the whole grid (the
// split count follows from the failure count, read on the device), write
// every score as an order-preserving key into the row's scratch slot and
// add the top-byte histogram of the row into its first digit histogram.  A
// row's score does not depend on its partner or its slot in the pair, so
// these are the walk's scores bit for bit.
constexpr int kPairFused = 0, kPairDebug = 1, kPairDense = 2, kPairControl = 3, kPairRepair = 4;

// Head-weighted sum of one row's 16 heads held by this lane plus its two
// u-block rows (ua, ub), in a fixed order (18 FMAs).
__device__ __forceinline__ float pair_epi(const float (&wh)[16], const float (&shr)[2], const v4f (&a)[4], float ua,
                                          float ub) {
  float x = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) x = fmaf(wh[4 * b + r], fabsf(a[b][r]), x);
  x = fmaf(shr[0], ua, x);
  return fmaf(shr[1], ub, x);
}

// Both rows' scores of one tile (lane l: key l, key scale applied) with the
// walk's arithmetic, unpipelined: the fused sampler's scores equal the
// walk's bit for bit.
__device__ __forceinline__ void pair_scores(const QOp2& qo, const KeyTile& kt, float& s0, float& s1) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  float q0[4], q1[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v4f aA[4], aB[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
      aA[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[0][b], kt.kb[c], z, 0, 0, 0, 0, 0, 0);
    const v4f au = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.au, kt.kb[c], z, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      aB[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[1][b], kt.kb[c], z, 0, 0, 0, 0, 0, 0);
    q0[c] = pair_epi(qo.wh[0], qo.sh[0], aA, au[0], au[1]);
    q1[c] = pair_epi(qo.wh[1], qo.sh[1], aB, au[2], au[3]);
  }
  s0 = reduce_scatter4(q0[0], q0[1], q0[2], q0[3]) * kt.ks;
  s1 = reduce_scatter4(q1[0], q1[1], q1[2], q1[3]) * kt.ks;
}

template <int MODE, bool SH = false, bool DIRECT = false>
__global__ __launch_bounds__(kWG, 2) void k_prefill_pair(PrefillArgs A) {
  static_assert(!SH || MODE != kPairRepair, "repair mode walks one pair per workgroup");
  static_assert(!SH || !DIRECT, "the shared walk reads the relaid copy");
  // key tiles from the relaid copy kt, or (DIRECT: calls too short to pay
  // for the copy) from k itself
  constexpr bool kRaw = DIRECT;
  __shared__ uint8_t s_qprep[kWaves][2 * kUTerms * kD];
  // optional clock probe: this wave's shader-clock cycles and constant-rate
  // wall-clock ticks from its start to its end, summed over all waves
  uint64_t clk0 = 0, rtc0 = 0;
  if (MODE != kPairRepair && A.clock) {
    clk0 = __builtin_amdgcn_s_memtime();
    rtc0 = __builtin_amdgcn_s_memrealtime();
  }
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if constexpr (MODE == kPairFused || MODE == kPairDebug) {
    // the first kernel of the call: the counters and the repair state start
    // at zero (read only by the kernels after this one)
    if (A.clear_main) {
      if (blockIdx.x == 0) clear_ctrl(A.ctrl, tid);
      if (!A.keep_all) {
        const int64_t i0 = (int64_t)blockIdx.x * kWG + tid, stride = (int64_t)gridDim.x * kWG;
        for (int64_t i = i0; i < (int64_t)A.rslots * kRepairDigits * 256; i += stride) A.rhist[i] = 0u;
        for (int64_t i = i0; i < (int64_t)A.rslots * kRowWords; i += stride) A.rrow[i] = 0u;
      }
    }
  }
  // the pair's rows (t_of: -1 for none) and, in repair mode, their scratch slots
  int split, nsplit, t_of[2], slot[2] = {0, 0};
  if constexpr (MODE == kPairRepair) {
    const int n_slot = (int)min(__atomic_load_n(&A.ctrl[kCtrlFail], __ATOMIC_RELAXED), (uint32_t)A.rslots);
    const int pairs = (n_slot + 1) / 2;
    if (pairs == 0) return;  // nothing failed (the whole workgroup leaves together)
    // splits per pair: the pairs fill one round of kRepairWalkWGs resident
    // workgroups (two per CU); the launch has a workgroup for every slot
    // pair, and those beyond the pairs' splits leave at once
    nsplit = max(1, kRepairWalkWGs / pairs);
    const int pr = blockIdx.x / nsplit;
    if (pr >= pairs) return;
    split = blockIdx.x % nsplit;
    slot[0] = 2 * pr;
    slot[1] = 2 * pr + 1;
    t_of[0] = A.fail_list[slot[0]];
    t_of[1] = slot[1] < n_slot ? A.fail_list[slot[1]] : -1;
  } else {
    nsplit = A.S;
    split = blockIdx.x % A.S;  // which share of the rows' tiles
    const int tb = SH ? kWaves * 2 * (blockIdx.x / A.S) + 2 * wave : 2 * (blockIdx.x / A.S);
    t_of[0] = tb < A.Q ? tb : -1;
    t_of[1] = tb + 1 < A.Q ? tb + 1 : -1;
  }
  const int tq = t_of[0] >= 0 ? t_of[0] : A.Q - 1;  // a real row for loads of an absent pair
  // this wave's segment of each row: one per split when the waves share
  // tiles (each walks all of them for its own pair), else one per wave
  const int seg = SH ? split : split * kWaves + wave;
  const int nseg = SH ? nsplit : kWaves * nsplit;

  int rs[2], re[2];
  float tr[2];
  int lo = 0x7fffffff, hi = -1;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    rs[r] = 0; re[r] = 0; tr[r] = INFINITY;
    const int t = t_of[r];
    if (t >= 0 && t < A.Q) {
      const int s = A.row_start[t], e = A.row_end[t];
      if (s >= 0 && s <= e && e <= A.N) {
        rs[r] = s; re[r] = e; tr[r] = (A.fuse_tau || A.keep_all) ? -INFINITY : A.tau[t];
        if (e > s) { lo = min(lo, s); hi = max(hi, e); }
      }
    }
  }
  __shared__ uint32_t s_rhist[2][256];  // repair: the pair's top-byte histograms
  if constexpr (MODE == kPairRepair) {
    s_rhist[0][tid] = 0u;
    s_rhist[1][tid] = 0u;
  }
  __shared__ int s_lohi[kWaves][2];
  if (SH && lane == 0) {
    s_lohi[wave][0] = lo;
    s_lohi[wave][1] = hi;
  }
  QOp2 qo;
  prepare_q2(qo, A.q, A.q_scale, A.w, tq, t_of[1] >= 0 ? t_of[1] : tq, lane, s_qprep[wave]);
  __syncthreads();
  if constexpr (SH) {  // the workgroup walks the union of its rows' ranges
    lo = min(min(s_lohi[0][0], s_lohi[1][0]), min(s_lohi[2][0], s_lohi[3][0]));
    hi = max(max(s_lohi[0][1], s_lohi[1][1]), max(s_lohi[2][1], s_lohi[3][1]));
  }
  // LDS shared by the sampler's scores and, after it, the staged key tiles
  // of the shared walk (two 8 KiB buffers)
  constexpr int kSampWords = (MODE == kPairFused || MODE == kPairDebug) ? (SH ? kWaves : 1) * 2 * kMaxSamples : 0;
  constexpr int kStageWords = SH ? 2 * kTile * kD / 4 : 0;
  __shared__ __attribute__((aligned(16))) uint32_t s_lds[kSampWords > kStageWords ? kSampWords : (kStageWords > 0 ? kStageWords : 1)];

  // Fused sampler ("3.2 Sampled threshold"), unless a threshold is forced:
  // the rows' thresholds are taken here, before the walk, instead of in a
  // kernel of their own (with S splits per row pair each split samples the
  // pair: the same values, in parallel; split 0 records them).  The waves
  // score the sampled keys' tiles (once for both rows when they share the
  // sample positions, as causal rows do) with the walk's arithmetic, so a
  // threshold is one of the walk's scores; wave r then selects row r's.
  // When the waves share tiles, each wave samples its own pair alone.
  if constexpr (MODE == kPairFused || MODE == kPairDebug) {
    if (A.fuse_tau) {
      uint32_t* const ss0 = s_lds + (SH ? wave : 0) * 2 * kMaxSamples;  // the rows' sampled scores
      uint32_t* const ss1 = ss0 + kMaxSamples;
      __shared__ uint32_t s_hist[SH ? kWaves : 2][256];
      __shared__ float s_tau[2];
      SampleGeom sg[2];
#pragma unroll
      for (int r = 0; r < 2; ++r)
        sg[r] = re[r] > rs[r] ? sample_geom(re[r] - rs[r], A.cand_cap) : SampleGeom{0, kSampleStride, 0};
      const KeyBuf kbuf = make_keybuf(A.k, A.k_scale, A.N);
      const auto pass = [&](int src, int n, bool st0, bool st1) {  // samples of row src's positions
#pragma unroll 1
        for (int i0 = SH ? 0 : kTile * wave; i0 < n; i0 += SH ? kTile : kTile * kWaves) {
          KeyTile kt;
          load_tile_gather(kt, kbuf, [&](int i) { return rs[src] + kSampleOffset + sg[src].stride * min(i0 + i, n - 1); },
                           lane);
          float s0, s1;
          pair_scores(qo, kt, s0, s1);
          const int i = i0 + (int)lane;
          if (st0 && i < sg[0].n) ss0[i] = f2key(s0);
          if (st1 && i < sg[1].n) ss1[i] = f2key(s1);
        }
      };
      if (sg[0].n > 0 && sg[1].n > 0 && rs[0] == rs[1] && sg[0].stride == sg[1].stride) {
        pass(0, max(sg[0].n, sg[1].n), true, true);
      } else {
        if (sg[0].n > 0) pass(0, sg[0].n, true, false);
        if (sg[1].n > 0) pass(1, sg[1].n, false, true);
      }
      if constexpr (SH) {
        wave_sync();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (sg[r].n > 0) {
            const SelResult sel = wave_radix_select(SrcLds{r == 0 ? ss0 : ss1}, sg[r].n, sg[r].r, s_hist[wave], lane, false);
            tr[r] = key2f(sel.prefix);
          }
        }
        __syncthreads();  // every wave is done with the sampler's LDS before tiles are staged there
      } else {
        __syncthreads();
        if (wave < 2) {
          const SampleGeom g = wave == 0 ? sg[0] : sg[1];
          if (g.n > 0) {
            const SelResult sel = wave_radix_select(SrcLds{wave == 0 ? ss0 : ss1}, g.n, g.r, s_hist[wave], lane, false);
            if (lane == 0) s_tau[wave] = key2f(sel.prefix);
          }
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 2; ++r)
          if (sg[r].n > 0) tr[r] = s_tau[r];  // else: -inf for a valid row (keeps all), +inf for an invalid one
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (split == 0 && (SH ? lane : tid) == r && t_of[r] >= 0) A.tau[t_of[r]] = tr[r];
    }
  }

  if constexpr (MODE == kPairFused || MODE == kPairDebug) {
    // keeping every key, the rows' thresholds are -inf (+inf for an invalid
    // range), recorded as the sampler records its thresholds
    if (A.keep_all) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (split == 0 && (SH ? lane : tid) == r && t_of[r] >= 0) A.tau[t_of[r]] = tr[r];
    }
  }

  const KeyBuf kbuf = make_keybuf(A.k, A.k_scale, A.N);
  const int ntiles = (A.N + 63) >> 6;
  // tile T's keys start at byte T*8192 in both layouts; block 2c+h of a tile
  // (bytes 32*(l/16) + 16h of key (sub-tile c, row l%16) for lane l) lies at
  // lane l's voff + boff(c, h) in the relaid copy, at gvoff + boff(c, h) in k
  const rsrc_t ktb = kRaw ? __builtin_amdgcn_make_buffer_rsrc((void*)A.k, (short)0, A.N * kD, 0x00020000)
                          : __builtin_amdgcn_make_buffer_rsrc((void*)A.kt, (short)0, ntiles * kTile * kD, 0x00020000);
  const uint32_t seg_cap = (uint32_t)A.seg_eff;
  const int tile_hi = (hi + 63) >> 6;
  const int voff = (int)lane * 16;  // LDS staging and relaid loads
  const int gvoff = kRaw ? (int)(lane & 15) * kD + 32 * (int)(lane >> 4) : voff;
  const auto boff = [](int c, int h) { return kRaw ? sub_off(c) * kD + 16 * h : (2 * c + h) * 1024; };
  uint32_t cnt[2] = {0u, 0u};  // candidates of each row found by this wave
  float csum[2] = {0.f, 0.f};  // control build: running sums of the rows' valid scores
  float dmax[2] = {-INFINITY, -INFINITY};  // per lane: largest candidate dropped for lack of room
  int fdrop[2] = {0x7FFFFFFF, 0x7FFFFFFF};  // position of the segment's first dropped candidate
  // the (row, wave) workspace segments as buffer resources: a store past
  // seg_cap is dropped by the bounds check
  rsrc_t segc[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int64_t o = MODE == kPairRepair ? 0 : ((int64_t)(t_of[r] >= 0 ? t_of[r] : tq) * nseg + seg) * A.seg_cap;
    segc[r] = __builtin_amdgcn_make_buffer_rsrc((void*)(A.cand + o), (short)0, (int)(seg_cap * 8u), 0x00020000);
  }
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  // Head-weighted sum of one row's 16 heads held by this lane plus its two
  // u-block rows (registers u0, u0+1 of the u accumulator), in a fixed order
  // (18 FMAs).
  const auto epi = [](const float (&wh)[16], const float (&shr)[2], const v4f (&a)[4], float ua, float ub) {
    return pair_epi(wh, shr, a, ua, ub);
  };
  // Per-tile state: row B's accumulators of the last sub-tile (its epilogue
  // runs under the next sub-tile's MFMAs) and the tile's partial sums.
  v4f aB[4] = {z, z, z, z}, auB = z;
  float q0[4], q1[4];
  // Tail of tile T: reduce-scatter, key scale, range and threshold tests,
  // append.  Branch-free: every lane stores, a taking lane at its slot in
  // the wave's segment (count + rank in the ballot), the others out of
  // range, where the buffer bounds check drops the store.  Candidates past
  // the segment's end are dropped the same way; the lanes that drop one
  // remember the largest dropped score (a rare, wave-uniform branch).
  const auto tail = [&](int T, float ks) {
    const float sc[2] = {reduce_scatter4(q0[0], q0[1], q0[2], q0[3]) * ks,
                         reduce_scatter4(q1[0], q1[1], q1[2], q1[3]) * ks};
    const int my = (T << 6) + (int)lane;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const bool valid = my >= rs[r] && my < re[r];
      if ((MODE == kPairDebug || MODE == kPairDense) && valid) A.dbg_scores[(int64_t)t_of[r] * A.N + my] = sc[r];
      if (MODE == kPairDense) continue;
      if (MODE == kPairControl) {
        csum[r] += valid ? sc[r] : 0.f;
        continue;
      }
      if (MODE == kPairRepair) {
        const uint32_t key = f2key(sc[r]);
        if (valid) A.scratch[(int64_t)slot[r] * A.rstride + (my - rs[r])] = key;
        hist_add(s_rhist[r], key >> 24, valid);
        continue;
      }
      const bool take = valid && sc[r] >= tr[r];
      const uint64_t ball = __ballot(take);
      const uint32_t n = (uint32_t)__popcll(ball);
      const int off = take ? (int)((cnt[r] + rank_in(ball)) * 8u) : 0x7FFFFFF0;
      const v2i cand = {(int)__float_as_uint(sc[r]), my};
      __builtin_amdgcn_raw_buffer_store_b64(cand, segc[r], off, 0, 0);
      if (cnt[r] + n > seg_cap) {
        const bool dropped = take && cnt[r] + rank_in(ball) >= seg_cap;
        dmax[r] = dropped ? fmaxf(dmax[r], sc[r]) : dmax[r];
        if (cnt[r] <= seg_cap) {  // the tile where the segment fills up
          int v = dropped ? my : 0x7FFFFFFF;
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
          fdrop[r] = __builtin_amdgcn_readfirstlane(v);
        }
      }
      cnt[r] += n;
    }
  };
  // One tile, software-pipelined by row across its sub-tiles.  Per 16-key
  // sub-tile c: row A's 4 MFMAs and the shared u MFMA, interleaved with row
  // B's epilogue of sub-tile c-1; then row B's 4 MFMAs, interleaved with row
  // A's epilogue of sub-tile c.  Row B's epilogue of the last sub-tile and
  // the tile's tail follow under row B's last MFMAs.  Once both rows' MFMAs
  // on sub-tile c are issued, its registers are refilled with the same
  // sub-tile of tile T+4 (a whole tile of lead from a single buffer); reads
  // past the end return 0.  (Carrying this pipeline across tiles measured
  // faster in isolation but does not fit the register budget of two
  // workgroups per CU.)
  //
  // Wave priority: raised over the sub-tiles (MFMAs with the epilogues
  // interleaved), normal for the tail, so that of the two waves on a SIMD
  // the one with MFMAs to issue goes first while the other finishes its
  // tail (3-4% faster than equal priorities).
  v8i kb[4];
  float ks_cur = 0.f;
  auto tile_body = [&](int T) {
    const int nT = refill_tile(T + nseg, ntiles);  // the tile refilled into kb
    const int ntoff = nT * (kTile * kD);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v4f aA[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        aA[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[0][b], kb[c], z, 0, 0, 0, 0, 0, 0);
      const v4f au = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.au, kb[c], z, 0, 0, 0, 0, 0, 0);
      if (c > 0) q1[c - 1] = epi(qo.wh[1], qo.sh[1], aB, auB[2], auB[3]);
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        aB[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[1][b], kb[c], z, 0, 0, 0, 0, 0, 0);
      kb[c] = cat8(__builtin_amdgcn_raw_buffer_load_b128(ktb, gvoff, ntoff + boff(c, 0), 0),
                   __builtin_amdgcn_raw_buffer_load_b128(ktb, gvoff, ntoff + boff(c, 1), 0));
      q0[c] = epi(qo.wh[0], qo.sh[0], aA, au[0], au[1]);
      auB = au;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    q1[3] = epi(qo.wh[1], qo.sh[1], aB, auB[2], auB[3]);
    tail(T, ks_cur);
    // The next tile's key scale is loaded only now, into the register the
    // tail just read: a load whose result were copied at the loop's back edge
    // would make that edge wait for every load issued before it (the memory
    // counter retires in order), that is for the whole next tile's keys.
    ks_cur = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kbuf.ks, (int)lane * 4, nT * 256, 0));
  };
  // The shared walk: the four waves score every tile of the split for
  // their own pairs, so each tile is read from memory once per workgroup.
  // Wave w stages blocks 2w and 2w+1 of the next tile into the free LDS
  // buffer: its loads go out at the start of the tile and land under the
  // tile's MFMAs; after the MFMAs it writes them, and one barrier, which
  // waits for LDS traffic only, hands the buffer over.  The next tile's B
  // operands are then read from LDS while the tail runs.
  const auto tile_body_shared = [&](int T, uint8_t* nxt) {
    const int nT = refill_tile(T + nseg, ntiles);
    const int ntoff = nT * (kTile * kD);
    const v4i g0 = __builtin_amdgcn_raw_buffer_load_b128(ktb, gvoff, ntoff + boff(wave, 0), 0);
    const v4i g1 = __builtin_amdgcn_raw_buffer_load_b128(ktb, gvoff, ntoff + boff(wave, 1), 0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v4f aA[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        aA[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[0][b], kb[c], z, 0, 0, 0, 0, 0, 0);
      const v4f au = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.au, kb[c], z, 0, 0, 0, 0, 0, 0);
      if (c > 0) q1[c - 1] = epi(qo.wh[1], qo.sh[1], aB, auB[2], auB[3]);
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        aB[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.a[1][b], kb[c], z, 0, 0, 0, 0, 0, 0);
      q0[c] = epi(qo.wh[0], qo.sh[0], aA, au[0], au[1]);
      auB = au;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    q1[3] = epi(qo.wh[1], qo.sh[1], aB, auB[2], auB[3]);
    *reinterpret_cast<v4i*>(nxt + (2 * wave) * 1024 + voff) = g0;
    *reinterpret_cast<v4i*>(nxt + (2 * wave + 1) * 1024 + voff) = g1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kb[c] = cat8(*reinterpret_cast<const v4i*>(nxt + (2 * c) * 1024 + voff),
                   *reinterpret_cast<const v4i*>(nxt + (2 * c + 1) * 1024 + voff));
    tail(T, ks_cur);
    ks_cur = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kbuf.ks, (int)lane * 4, nT * 256, 0));
  };
  if constexpr (SH) {
    if (lo < hi) {  // uniform over the workgroup
      int T = (lo >> 6) + seg;
      uint8_t* const buf0 = reinterpret_cast<uint8_t*>(s_lds);
      {
        const int t1 = refill_tile(T, ntiles);  // past the last tile: the loop is empty
        const int toff = t1 * (kTile * kD);
        *reinterpret_cast<v4i*>(buf0 + (2 * wave) * 1024 + voff) =
            __builtin_amdgcn_raw_buffer_load_b128(ktb, gvoff, toff + boff(wave, 0), 0);
        *reinterpret_cast<v4i*>(buf0 + (2 * wave + 1) * 1024 + voff) =
            __builtin_amdgcn_raw_buffer_load_b128(ktb, gvoff, toff + boff(wave, 1), 0);
        ks_cur = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kbuf.ks, (int)lane * 4, t1 * 256, 0));
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < 4; ++c)
        kb[c] = cat8(*reinterpret_cast<const v4i*>(buf0 + (2 * c) * 1024 + voff),
                     *reinterpret_cast<const v4i*>(buf0 + (2 * c + 1) * 1024 + voff));
      int b = kTile * kD;  // offset of the buffer the next tile is staged in
#pragma unroll 1
      for (; T < tile_hi; T += nseg, b ^= kTile * kD) tile_body_shared(T, buf0 + b);
    }
  } else if (lo < hi) {
    int T = (lo >> 6) + seg;
    {
      const int t0 = refill_tile(T, ntiles);  // past the last tile: the loop is empty
#pragma unroll
      for (int c = 0; c < 4; ++c)
        kb[c] = cat8(__builtin_amdgcn_raw_buffer_load_b128(ktb, gvoff, t0 * (kTile * kD) + boff(c, 0), 0),
                     __builtin_amdgcn_raw_buffer_load_b128(ktb, gvoff, t0 * (kTile * kD) + boff(c, 1), 0));
      ks_cur = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kbuf.ks, (int)lane * 4, t0 * 256, 0));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // drain once so the loop's waits stay exact
#pragma unroll 1
    for (; T < tile_hi; T += nseg) tile_body(T);
  }

  if constexpr (MODE == kPairControl) {
    // the checksums go to the unused fourth word of the segment records
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float m = csum[r];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m += __shfl_xor(m, o, 64);
      if (lane == 0 && t_of[r] >= 0) A.segn[4 * ((int64_t)t_of[r] * nseg + seg) + 3] = __float_as_uint(m);
    }
  } else if constexpr (MODE == kPairRepair) {
    // the pair's histograms into the rows' first digit histograms
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t h = s_rhist[r][tid];
      if (h && t_of[r] >= 0) atomicAdd(&A.rhist[(int64_t)slot[r] * kRepairDigits * 256 + tid], h);
    }
  } else if constexpr (MODE != kPairDense) {
    // publish this wave's segment: entries stored, the order-preserving key of
    // the largest dropped candidate (0: none dropped; a candidate is never
    // NaN, so its key is nonzero) and the position of the first dropped one
    // (candidates arrive in position order, so every later one was dropped)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint32_t dk = 0u;
      if (cnt[r] > seg_cap) {
        float m = dmax[r];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        dk = f2key(m);
      }
      if (lane == 0 && t_of[r] >= 0)
        *reinterpret_cast<uint4*>(A.segn + 4 * ((int64_t)t_of[r] * nseg + seg)) =
            make_uint4(min(cnt[r], seg_cap), dk, (uint32_t)fdrop[r], 0u);
    }
  }
  if (MODE != kPairRepair && A.clock && lane == 0) {
    atomicAdd(reinterpret_cast<unsigned long long*>(A.clock), (unsigned long long)(__builtin_amdgcn_s_memtime() - clk0));
    atomicAdd(reinterpret_cast<unsigned long long*>(A.clock + 1),
              (unsigned long long)(__builtin_amdgcn_s_memrealtime() - rtc0));
  }
}

// ------------------------------------------------------------------ select

// One workgroup per row, after the main kernel.  The row's candidates (its
// nseg segments: segment g in threads [g*tps, (g+1)*tps), tps = 64*NW/nseg,
// each thread every tps-th entry, M slots per thread) are loaded into registers and
// the K largest selected, ties at the K-th score going to the lowest ids.
// Certificate ("3.2 Sampled threshold", made exact for capacity drops):
// this is the row's exact top-K iff there were at least K candidates and
// no dropped candidate scores above the smallest selected score theta; if
// a dropped one equals theta, the tied ids taken must also all lie below
// the first dropped position (segments drop only their latest candidates),
// so that they are the lowest tied ids of the whole row.  Massive ties at
// the boundary thus need no repair.  Rows that fail go to the failure list.
// NW waves per workgroup: 4 where many rows share each CU, 16 (four times
// fewer slots per thread, so shorter chains) for calls with few rows.
template <int M, int NW>
__global__ __launch_bounds__(64 * NW) void k_prefill_select(PrefillArgs A) {
  constexpr int NT = 64 * NW;
  __shared__ SelShared sh;
  __shared__ uint32_t s_segn[kWaves * kMaxSplit];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int t = blockIdx.x;
  uint32_t* stats = stat_copy(A.ctrl, blockIdx.x);
  int32_t* out = A.out + (int64_t)t * A.K;
  if (tid == 0) atomicAdd(&stats[kStRows], 1u);
  // the segment records are loaded beside the row's range (one round trip
  // for both; for an invalid row they are read and unused)
  const int nseg = A.nseg;
  uint4 e = make_uint4(0u, 0u, 0u, 0u);
  if (tid < nseg) e = *reinterpret_cast<const uint4*>(A.segn + 4 * ((int64_t)t * nseg + tid));
  const int rs_t = A.row_start[t], re_t = A.row_end[t];
  if (rs_t < 0 || rs_t > re_t || re_t > A.N) {
    for (int i = tid; i < A.K; i += NT) out[i] = -1;
    if (tid == 0) {
      atomicAdd(&stats[kStBad], 1u);
      if (A.row_status) A.row_status[t] = IDX_ROW_BAD;
    }
    return;
  }
  uint32_t dk = 0u, fd = 0xFFFFFFFFu;
  if (tid < nseg) {
    s_segn[tid] = e.x;
    dk = e.y;
    fd = e.y ? e.z : 0xFFFFFFFFu;
  }
  // largest dropped key and first dropped position over the segments (all
  // in wave 0: nseg <= 32)
  dk = wave_max_u32(dk);
  fd = wave_min_u32(fd);
  if (tid == 0) { sh.pad0 = dk; sh.pad1 = fd; }
  __syncthreads();
  const uint32_t drop = sh.pad0, first_drop = sh.pad1;
  uint32_t n = 0u, most = 0u;  // candidates in all, in the fullest segment
  for (int g = 0; g < nseg; ++g) {
    n += s_segn[g];
    most = max(most, s_segn[g]);
  }
  const int L = re_t - rs_t;
  const int kr = min(A.K, L);
  bool ok = n >= (uint32_t)kr;
  if (ok) {
    const uint32_t tps = (uint32_t)(NT / nseg);
    const uint32_t g = (uint32_t)tid / tps;
    const uint32_t first = g * (uint32_t)A.seg_cap;
    // slots past the fullest segment's entries are empty in every thread:
    // the select's loops stop there
    const uint32_t jmax = min((most + tps - 1u) / tps, (uint32_t)M);
    const RegLayout lay{first + (uint32_t)tid % tps, tps, first + s_segn[g], jmax};
    const int64_t row = (int64_t)t * nseg * A.seg_cap;
    uint32_t key[M];
    int32_t id[M];
    load_list_regs(key, id, A.cand + row, (uint32_t)(nseg * A.seg_cap), lay,
                   [](uint32_t x) { return f2key(__uint_as_float(x)); });
    const auto kf = [&](int j) { return key[j]; };
    const RangeSel sel = (n > (uint32_t)kr) ? range_select_regs<M, NW>(kf, lay, kr, sh, tid)
                                           : RangeSel{1u, 0xFFFFFFFFu, kr, (int)n};
    const uint32_t idlo = tie_bound_regs<NW>(key, id, lay, sel, sh, tid);
    if (drop >= sel.lo) {
      const uint32_t theta = range_min_regs<M, NW>(kf, lay, sel, sh, tid);
      ok = drop <= theta;
      if (drop == theta) {  // tied keys were dropped: the taken ones must precede them
        const auto tk = [&](int j) {  // recomputed per use (see tie_bound_regs)
          uint32_t x = (uint32_t)id[j];
          asm volatile("" : "+v"(x));
          return key[j] == theta && ~x >= idlo ? ~x : 0xFFFFFFFFu;
        };
        uint32_t mn = 0xFFFFFFFFu;  // smallest ~id taken at theta = ~(largest id)
#pragma unroll
        for (int j = 0; j < M; ++j) mn = min(mn, tk(j));
        mn = wave_min_u32(mn);
        if (lane == 0) sh.wsum[0][tid >> 6] = mn;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w) mn = min(mn, sh.wsum[0][w]);
        __syncthreads();
        ok = ok && ~mn < first_drop;
      }
    }
    if (ok) emit_range_regs<NW>(key, id, lay, sel, idlo, kr, A.K, out, IdIdentity{}, sh, tid);
  }
  if (tid == 0) {
    if (A.row_status) A.row_status[t] = ok ? IDX_ROW_FAST : drop ? IDX_ROW_OVERFLOW : IDX_ROW_UNDERFLOW;
    if (ok) {
      atomicAdd(&stats[kStFast], 1u);
      if (n > (uint32_t)kManyCands) atomicAdd(&stats[kStMany], 1u);
      if (L <= A.K) atomicAdd(&stats[kStTrivial], 1u);
    } else {
      const uint32_t f = atomicAdd(&A.ctrl[kCtrlFail], 1u);
      A.fail_list[f] = t;
      atomicAdd(&stats[drop ? kStOver : kStUnder], 1u);
    }
  }
}

// ------------------------------------------------------------------ repair
//
// Exact repair of rows the certificate rejected, split over the whole chip:
// the first rslots failed rows each get a scratch slot, and the kernels
// below walk work items (f, c) = (failed row, chunk of kRepairChunk
// positions), each workgroup a contiguous run of them, so that its items
// mostly share a row.  The radix select runs one 8-bit digit per launch:
// the digit histogram of a row is summed in device memory over its chunks;
// the next launch advances the row's selection state by that digit (once
// per row and workgroup, from the state the launch before stored) and its
// chunk-0 item stores the result for the launch after.  The two digits'
// states go to two word groups, so a launch never overwrites the one it
// reads.  After two digits the gather writes out every key above the
// boundary prefix and collects the boundary group; the final kernel, one
// workgroup per row, selects the rest of the row's top-K among them.

struct RepairSel {
  uint32_t prefix, mask;
  int rem;
  int group;  // keys with (key & mask) == prefix
  bool done;  // the boundary group is taken whole (rem == group)
};

__device__ __forceinline__ RepairSel load_state(const uint32_t* rw, int buf) {
  const uint32_t* w = rw + kRowState + 4 * buf;
  const bool done = w[3] == 0xFFFFFFFFu;
  return RepairSel{w[0], w[1], (int)w[2], done ? (int)w[2] : (int)w[3], done};
}

__device__ __forceinline__ void store_state(uint32_t* rw, int buf, const RepairSel& s) {
  *reinterpret_cast<uint4*>(rw + kRowState + 4 * buf) =
      make_uint4(s.prefix, s.mask, (uint32_t)s.rem, s.done ? 0xFFFFFFFFu : (uint32_t)s.group);
}

// A chunk kernel's current row: its id, range, keys kept and selection state.
struct RepairRow {
  int f, t, s0, L, kr;
  RepairSel sel;
};

__device__ __forceinline__ void repair_row_ids(RepairRow& row, const PrefillArgs& A, int f) {
  row.f = f;
  row.t = A.fail_list[f];
  row.s0 = A.row_start[row.t];
  row.L = A.row_end[row.t] - row.s0;
  row.kr = min(A.K, row.L);
}

// Load slot f's row and its selection state after `digits` digits (1 or
// 2): the state after digits-1 (the initial one for digits == 1, else as
// the previous launch stored it) advanced by that digit's complete
// histogram.  Whole workgroup calls.
__device__ void repair_row_at(RepairRow& row, const PrefillArgs& A, int f, int digits, SelShared& sh, int tid) {
  repair_row_ids(row, A, f);
  const uint32_t* rw = A.rrow + (int64_t)f * kRowWords;
  RepairSel s = digits == 1 ? RepairSel{0u, 0u, row.kr, row.L, row.L <= row.kr} : load_state(rw, (digits - 1) & 1);
  if (!s.done) {
    __syncthreads();  // the previous item's reads of sh are done
    sh.hist[tid] = A.rhist[((int64_t)f * kRepairDigits + digits - 1) * 256 + tid];
    __syncthreads();
    find_bucket(sh, s.rem, tid);
    __syncthreads();
    const int shift = 32 - 8 * digits;
    s.prefix |= sh.bucket << shift;
    s.mask |= 0xFFu << shift;
    s.rem -= (int)sh.above;
    s.group = (int)sh.inbucket;
    s.done = s.group == s.rem;
  }
  row.sel = s;
}

// Contiguous run of the n items for this workgroup.
__device__ __forceinline__ void item_run(int64_t n, int64_t& i0, int64_t& i1) {
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  i0 = min(n, per * (int64_t)blockIdx.x);
  i1 = min(n, i0 + per);
}

// Failures beyond the repair slots (the slotted ones are rescored by the
// main kernel's repair mode) are repaired whole, one per fallback
// workgroup.
__global__ __launch_bounds__(kWG) void k_prefill_repair_fallback(PrefillArgs A) {
  __shared__ SelShared sh;
  __shared__ uint8_t s_qprep[kWaves][kUTerms * kD];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t n_fail = __atomic_load_n(&A.ctrl[kCtrlFail], __ATOMIC_RELAXED);
  if (blockIdx.x >= kRepairFallback) return;
  uint32_t* own = A.scratch + ((int64_t)A.rslots + blockIdx.x) * A.rstride;
  uint32_t* stats = stat_copy(A.ctrl, blockIdx.x);
#pragma unroll 1
  for (uint32_t f = (uint32_t)A.rslots + blockIdx.x; f < n_fail; f += kRepairFallback) {
    const int t = A.fail_list[f];
    const int s0 = A.row_start[t], s1 = A.row_end[t];
    QOp qo;
    prepare_q(qo, A.q, A.q_scale, A.w, t, lane, s_qprep[wave], t & 1);
    repair_row(qo, make_keybuf(A.k, A.k_scale, A.N), TileContig{}, IdIdentity{}, s0, s1, A.K,
               A.out + (int64_t)t * A.K, own, sh, tid);
    if (tid == 0) atomicAdd(&stats[kStRepaired], 1u);
    __syncthreads();
  }
}

// Keys of chunk c of a scratch row, four per 16-byte load: thread tid holds
// positions c*kRepairChunk + 4*(k*kWG + tid) + e for k < 4, e < 4.
struct ChunkKeys {
  uint32_t v[16];
  int base;  // position of v[0] relative to the row start
};

__device__ __forceinline__ void load_chunk(ChunkKeys& ck, const uint32_t* row, int c, int L, int tid) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e0 = c * kRepairChunk + 4 * (k * kWG + tid);
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (e0 < L) x = *reinterpret_cast<const uint4*>(row + e0);
    ck.v[4 * k + 0] = x.x; ck.v[4 * k + 1] = x.y; ck.v[4 * k + 2] = x.z; ck.v[4 * k + 3] = x.w;
  }
  ck.base = c * kRepairChunk + 4 * tid;
}

__device__ __forceinline__ int chunk_pos(const ChunkKeys& ck, int j) { return ck.base + (j >> 2) * 4 * kWG + (j & 3); }

// Second digit over the slotted failed rows that are still open: the
// histogram of bits 16..23 among the keys that share the K-th key's top
// byte.
__global__ __launch_bounds__(kWG) void k_prefill_repair_pass(PrefillArgs A) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const uint32_t n_slot = min(__atomic_load_n(&A.ctrl[kCtrlFail], __ATOMIC_RELAXED), (uint32_t)A.rslots);
  const int cmax = (A.N + kRepairChunk - 1) / kRepairChunk;
  int64_t i0, i1;
  item_run((int64_t)n_slot * cmax, i0, i1);
  RepairRow row;
  row.f = -1;
#pragma unroll 1
  for (int64_t i = i0; i < i1; ++i) {
    const int f = (int)(i / cmax), c = (int)(i % cmax);
    if (f != row.f) repair_row_at(row, A, f, 1, sh, tid);
    if (c == 0 && tid == 0) store_state(A.rrow + (int64_t)f * kRowWords, 1, row.sel);
    if (row.sel.done || c * kRepairChunk >= row.L) continue;
    ChunkKeys ck;
    load_chunk(ck, A.scratch + (int64_t)f * A.rstride, c, row.L, tid);
    __syncthreads();  // the previous item's reads of sh are done
    sh.hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool v = chunk_pos(ck, j) < row.L && (ck.v[j] & row.sel.mask) == row.sel.prefix;
      hist_add(sh.hist, (ck.v[j] >> 16) & 255u, v);
    }
    __syncthreads();
    const uint32_t h = sh.hist[tid];
    if (h) atomicAdd(&A.rhist[((int64_t)f * kRepairDigits + 1) * 256 + tid], h);
  }
}

// The failed row's candidate area holds its gathered boundary group:
// (key, id) pairs, at most kRepairGroupCap of them.
__device__ __forceinline__ uint2* repair_group(const PrefillArgs& A, int t) {
  return A.cand + (int64_t)t * A.nseg * A.seg_cap;
}

// After two digits: every key above the boundary prefix is written out
// (positions from the row's counter, in any order), and so is the boundary
// group when it is taken whole; otherwise the group is gathered for the
// final kernel, unless it exceeds kRepairGroupCap (massive ties), when the
// final kernel reads it from scratch instead.
__global__ __launch_bounds__(kWG) void k_prefill_repair_gather(PrefillArgs A) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const uint32_t n_slot = min(__atomic_load_n(&A.ctrl[kCtrlFail], __ATOMIC_RELAXED), (uint32_t)A.rslots);
  const int cmax = (A.N + kRepairChunk - 1) / kRepairChunk;
  int64_t i0, i1;
  item_run((int64_t)n_slot * cmax, i0, i1);
  uint32_t* stats = stat_copy(A.ctrl, blockIdx.x);
  RepairRow row;
  row.f = -1;
#pragma unroll 1
  for (int64_t i = i0; i < i1; ++i) {
    const int f = (int)(i / cmax), c = (int)(i % cmax);
    uint32_t* rw = A.rrow + (int64_t)f * kRowWords;
    if (f != row.f) repair_row_at(row, A, f, 2, sh, tid);
    const int s0 = row.s0, L = row.L, kr = row.kr;
    const RepairSel& rs = row.sel;
    int32_t* out = A.out + (int64_t)row.t * A.K;
    if (c == 0) {
      if (tid == 0) {
        store_state(rw, 0, rs);
        atomicAdd(&stats[kStRepaired], 1u);
      }
      for (int j = kr + tid; j < A.K; j += kWG) out[j] = -1;
    }
    if (c * kRepairChunk >= L) continue;
    ChunkKeys ck;
    load_chunk(ck, A.scratch + (int64_t)f * A.rstride, c, L, tid);
    const bool gather = !rs.done && rs.group <= kRepairGroupCap;  // uniform
    uint32_t gmask = 0u, emask = 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool v = chunk_pos(ck, j) < L;
      const uint32_t mk = ck.v[j] & rs.mask;
      gmask |= (uint32_t)(v && mk > rs.prefix) << j;
      emask |= (uint32_t)(v && mk == rs.prefix && (rs.done || gather)) << j;
    }
    // count this chunk's keys of each class in LDS, then reserve their
    // output range with one device-memory atomic per class
    __syncthreads();  // the previous item's reads of sh are done
    if (tid == 0) { sh.gt_count = 0u; sh.eq_count = 0u; }
    __syncthreads();
    const uint32_t ng = (uint32_t)__popc(gmask), ne = (uint32_t)__popc(emask);
    uint32_t pg = 0u, pe = 0u;
    if (ng) pg = atomicAdd(&sh.gt_count, ng);
    if (ne) pe = atomicAdd(&sh.eq_count, ne);
    __syncthreads();
    if (tid == 0) {
      sh.pad0 = sh.gt_count ? atomicAdd(&rw[kRowGt], sh.gt_count) : 0u;
      sh.pad1 = sh.eq_count ? atomicAdd(&rw[kRowEq], sh.eq_count) : 0u;
    }
    __syncthreads();
    pg += sh.pad0;
    pe += sh.pad1;
    const int eq_base = kr - rs.rem;
    uint2* grp = repair_group(A, row.t);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int pos = chunk_pos(ck, j);
      if (gmask >> j & 1u) out[pg++] = s0 + pos;
      if (emask >> j & 1u) {
        if (rs.done) {
          if ((int)pe < rs.rem) out[eq_base + pe] = s0 + pos;
        } else if ((int)pe < kRepairGroupCap) {
          grp[pe] = make_uint2(ck.v[j], (uint32_t)(s0 + pos));
        }
        ++pe;
      }
    }
  }
}

// A row's scratch keys restricted to its boundary group (0 elsewhere: below
// every key of the group, which are nonzero).
struct SrcGroup {
  const uint32_t* row;
  uint32_t mask, prefix;
  int s0;
  __device__ uint32_t key(int i) const {
    const uint32_t k = row[i];
    return (k & mask) == prefix ? k : 0u;
  }
  __device__ int32_t id(int i) const { return s0 + i; }
};

// One workgroup per slotted failed row still open after two digits: the
// rem largest of its boundary group, ties at the K-th score to the lowest
// ids, into out[kr - rem, kr).  A gathered group is selected in registers
// (range select, then the tie-break on the ids); a larger one by radix
// passes over the row's scratch keys, restricted to the group, whose emit
// takes tied keys in position order.
__global__ __launch_bounds__(64 * kMaxWaves) void k_prefill_repair_final(PrefillArgs A) {
  constexpr int NW = kMaxWaves;  // one row per workgroup: 1024 threads shorten its chains
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const uint32_t n_slot = min(__atomic_load_n(&A.ctrl[kCtrlFail], __ATOMIC_RELAXED), (uint32_t)A.rslots);
#pragma unroll 1
  for (uint32_t f = blockIdx.x; f < n_slot; f += gridDim.x) {
    RepairRow row;
    repair_row_ids(row, A, (int)f);
    const RepairSel rs = load_state(A.rrow + (int64_t)f * kRowWords, 0);
    if (rs.done) continue;  // written whole by the gather
    int32_t* out = A.out + (int64_t)row.t * A.K + (row.kr - rs.rem);
    if (rs.group <= kRepairGroupCap) {
      constexpr int M = kRepairGroupCap / (64 * NW);
      const uint32_t n = (uint32_t)rs.group;
      const RegLayout lay = block_list_layout<NW>(n, (uint32_t)tid);
      uint32_t key[M];
      int32_t id[M];
      load_list_regs(key, id, repair_group(A, row.t), n, lay, [](uint32_t x) { return x; });
      const auto kf = [&](int j) { return key[j]; };
      const RangeSel sel = range_select_regs<M, NW>(kf, lay, rs.rem, sh, tid);  // rem < group
      const uint32_t idlo = tie_bound_regs<NW>(key, id, lay, sel, sh, tid);
      emit_range_regs<NW>(key, id, lay, sel, idlo, rs.rem, rs.rem, out, IdIdentity{}, sh, tid);
    } else {
      const SrcGroup src{A.scratch + (int64_t)f * A.rstride, rs.mask, rs.prefix, row.s0};
      const SelResult sel = radix_select<NW>(src, row.L, rs.rem, sh, tid, false, true);
      emit_selection<NW>(src, row.L, sel, rs.rem, rs.rem, out, sh, tid);
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ launch

// One launch of the main kernel in mode MODE with the call's walk geometry
// and key source; the events, when given, are recorded by the launch itself.
template <int MODE>
static void launch_main(const PrefillArgs& A, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int rows = A.shared ? kSharedRows : 2;
  const unsigned grid = (unsigned)((A.Q + rows - 1) / rows * A.S);
  void (*const kern)(PrefillArgs) = A.shared   ? k_prefill_pair<MODE, true>
                                    : A.direct ? k_prefill_pair<MODE, false, true>
                                               : k_prefill_pair<MODE, false, false>;
  if (e0 || e1)
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(kWG), 0, stream, e0, e1, 0, A);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kWG), 0, stream, A);
}

// The relaid key copy is made for every call but the one-pair walk over
// calls that keep every key (A.direct): those are too short to pay for the
// copy's launch, while elsewhere reading k itself cost the main kernel more
// than the copy (the one-pair walk 20-25%, the shared walk 8% more cycles).
// Without the relayout kernel the main kernel takes over its other duties.
int launch_prefill(const PrefillArgs& args, hipStream_t stream) {
  if (args.Q == 0) return IDX_OK;
  PrefillArgs A = args;
  const int64_t nchunks = (int64_t)((A.N + 63) >> 6) * 512;
  if (!A.direct && nchunks > 0)
    hipLaunchKernelGGL(k_relayout_keys, dim3((unsigned)(nchunks / kWG)), dim3(kWG), 0, stream, A);
  else
    A.clear_main = (A.keep_all || A.fuse_tau) ? 1 : 0;  // k_prefill_tau is not launched either
  if (A.math_only) {  // the control: the main kernel's scoring alone, nothing after it
    const int reps = A.main_reps > 1 ? A.main_reps : 1;
    for (int r = 0; r < reps; ++r)
      launch_main<kPairControl>(A, stream, r == 0 ? A.ev_main_start : nullptr,
                                r == reps - 1 ? A.ev_main_stop : nullptr);
    return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
  }
  if (!A.keep_all && !A.fuse_tau) hipLaunchKernelGGL(k_prefill_tau, dim3(kRepairGrid), dim3(kWG), 0, stream, A);
  // the timing events, when given, are recorded by the launches themselves
  // (the first launch's start, the last launch's end; main_reps > 1 repeats
  // the idempotent kernel for timing); without events a plain launch (the
  // extended one measured up to 1% slower per call)
  const int reps = A.main_reps > 1 ? A.main_reps : 1;
  for (int r = 0; r < reps; ++r) {
    hipEvent_t e0 = r == 0 ? A.ev_main_start : nullptr, e1 = r == reps - 1 ? A.ev_main_stop : nullptr;
    if (A.dbg_scores)
      launch_main<kPairDebug>(A, stream, e0, e1);
    else
      launch_main<kPairFused>(A, stream, e0, e1);
  }
  // calls with few rows: 1024 threads per row; otherwise 256, and candidate
  // slots per thread a segment's capacity over its threads (256 / nseg of
  // them): 33 for one, two or four segments per row, up to 40 for 8..32
  // (fewer registers let more rows run at once)
  if (A.Q <= kSelWideRows)
    hipLaunchKernelGGL((k_prefill_select<kSelRegsWide, kMaxWaves>), dim3(A.Q), dim3(64 * kMaxWaves), 0, stream, A);
  else if (A.nseg <= 4)
    hipLaunchKernelGGL((k_prefill_select<kSelRegsFew, kWaves>), dim3(A.Q), dim3(kWG), 0, stream, A);
  else
    hipLaunchKernelGGL((k_prefill_select<kSelRegs, kWaves>), dim3(A.Q), dim3(kWG), 0, stream, A);
  if (A.keep_all) return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;  // nothing can need repair
  // the slotted failures rescored two per workgroup: enough workgroups for
  // every slot pair, at least two per CU for few failures
  const unsigned rgrid = (unsigned)max(kRepairWalkWGs, (A.rslots + 1) / 2);
  if (A.direct)
    hipLaunchKernelGGL((k_prefill_pair<kPairRepair, false, true>), dim3(rgrid), dim3(kWG), 0, stream, A);
  else
    hipLaunchKernelGGL((k_prefill_pair<kPairRepair, false, false>), dim3(rgrid), dim3(kWG), 0, stream, A);
  if (A.rslots < A.Q) hipLaunchKernelGGL(k_prefill_repair_fallback, dim3(kRepairFallback), dim3(kWG), 0, stream, A);
  hipLaunchKernelGGL(k_prefill_repair_pass, dim3(kRepairPassGrid), dim3(kWG), 0, stream, A);
  hipLaunchKernelGGL(k_prefill_repair_gather, dim3(kRepairPassGrid), dim3(kWG), 0, stream, A);
  hipLaunchKernelGGL(k_prefill_repair_final, dim3((unsigned)min(A.rslots, kRepairFinalGrid)), dim3(64 * kMaxWaves), 0,
                     stream, A);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

// Unfused comparator ("2.2 Indexer scoring is compute-bound", "6.2 Operator
// performance"): the same MFMA scoring
// writes the whole [Q,N] FP32 score matrix to A.dbg_scores, then the
// dense-matrix top-K selects each row from it.  The sampler kernel runs
// only to clear the control words (its forced threshold is unused).
int launch_prefill_unfused(const PrefillArgs& A, hipStream_t stream) {
  if (A.Q == 0) return IDX_OK;
  const int64_t nchunks = (int64_t)((A.N + 63) >> 6) * 512;
  if (!A.direct && nchunks > 0)
    hipLaunchKernelGGL(k_relayout_keys, dim3((unsigned)(nchunks / kWG)), dim3(kWG), 0, stream, A);
  hipLaunchKernelGGL(k_prefill_tau, dim3(kRepairGrid), dim3(kWG), 0, stream, A);
  const int reps = A.main_reps > 1 ? A.main_reps : 1;
  for (int r = 0; r < reps; ++r)
    launch_main<kPairDense>(A, stream, r == 0 ? A.ev_main_start : nullptr, r == reps - 1 ? A.ev_main_stop : nullptr);
  if (hipGetLastError() != hipSuccess) return IDX_EHIP;
  RowsArgs R{A.dbg_scores, (int64_t)A.N, A.row_start, A.row_end, A.Q, A.N, A.K, A.out, A.ctrl};
  return launch_topk_rows(R, stream);
}

}  // namespace idxk
