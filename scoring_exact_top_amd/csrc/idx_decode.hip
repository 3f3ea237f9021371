// Paged decode path (contest report page (arXiv 2608.14560), "DSA TopK Indexer"): one FP8 query
// per sequence against its keys in a paged FP8 cache with per-token scales.
//
//   k_decode_prep   one sequence per wave: validate the sequence's page
//                   ids; sequences with seq_len <= K take the remap path
//                   (every slot is selected, no scoring); longer ones get a
//                   sampled threshold.
//   k_decode_split  G workgroups per sequence split its keys (KV-dimension
//                   parallelism, Fusing Indexer Scoring and Exact Top-k
//                   page, "10. The optimization target after fusion"); each
//                   scores its chunk and appends keys >= tau to the
//                   sequence's candidate list in the workspace.
//   k_decode_select one workgroup per sequence: certificate, register-
//                   resident radix select, emit.  A kernel boundary rather
//                   than an in-kernel last-arriver handoff: on this chip the
//                   device-scope fence such a handoff needs writes back and
//                   invalidates the L2 of the XCD, once per workgroup.
//                   No host synchronisation anywhere.
//   k_decode_repair exact repair of sequences the certificate rejected.
#include <string.h>

#include "idx_decode.hpp"
#include "idx_internal.hpp"

namespace idxk {

constexpr int kDecCap = 8192;    // candidate list capacity per sequence
constexpr int kDecStage = 512;   // per-wave LDS stage of the split kernel

struct DecodeArgs {
  const uint8_t* q;
  const float* q_scale;
  const uint8_t* k;      // [num_pages*64][128]
  const float* k_scale;  // [num_pages*64]
  const float* w;
  const int32_t* table;  // [B][max_pages]
  const int32_t* seq_lens;
  int32_t B, max_pages, num_pages, K, G;
  int32_t* out;          // [B][K]
  uint32_t* ctrl;
  float* tau;            // [B]
  int32_t* status;       // [B]: 0 score, 1 remapped, 2 invalid
  uint32_t* cnt;         // [B] candidates appended (may exceed kDecCap)
  uint32_t* drop;        // [B][2]: key of the largest dropped candidate (0: none), lowest dropped position
  int32_t* fail_list;    // [B]
  uint32_t* cand_key;    // [B][kDecCap] candidate scores (FP32 bits)
  int32_t* cand_idx;     // [B][kDecCap] candidate logical positions
  uint32_t* scratch;     // [repair_grid(B)][max_pages*64]
  uint32_t* qop;         // [B][kQOpWords][64] prepared query operands
  int32_t force_tau;     // debug: every scored sequence uses tau_value
  float tau_value;
};

// One sequence per wave: validate its page ids, remap when L <= K, else
// draw its sampled threshold (the prefill sampler's lattice and estimator).
__global__ __launch_bounds__(kWG) void k_decode_prep(DecodeArgs A) {
  __shared__ uint32_t s_samp[kWaves][kMaxSamples];
  __shared__ uint32_t s_hist[kWaves][256];
  __shared__ uint8_t s_qprep[kWaves][kUTerms * kD];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (blockIdx.x == 0) clear_ctrl(A.ctrl, tid);
  const int b = kWaves * blockIdx.x + wave;
  if (b >= A.B) return;
  if (lane == 0) {
    A.cnt[b] = 0u;
    A.drop[2 * b] = 0u;
    A.drop[2 * b + 1] = 0xFFFFFFFFu;
  }
  const int L = A.seq_lens[b];
  const int32_t* pt = A.table + (int64_t)b * A.max_pages;
  int32_t* out = A.out + (int64_t)b * A.K;
  bool bad = L < 0 || L > A.max_pages * 64;
  if (!bad) {
    for (int p = (int)lane; p < ((L + 63) >> 6); p += 64) {
      const int pg = pt[p];
      bad |= pg < 0 || pg >= A.num_pages;
    }
  }
  if (__ballot(bad)) {
    for (int i = (int)lane; i < A.K; i += 64) out[i] = -1;
    if (lane == 0) A.status[b] = 2;
    return;
  }
  if (L <= A.K) {
    // every position is in the top-K: remap to physical slots
    for (int i = (int)lane; i < A.K; i += 64) out[i] = i < L ? pt[i >> 6] * 64 + (i & 63) : -1;
    if (lane == 0) A.status[b] = 1;
    return;
  }
  // the query operands, prepared once here for every workgroup of the split
  QOp qo;
  prepare_q(qo, A.q, A.q_scale, A.w, b, lane, s_qprep[wave], 0);
  store_qop(qo, A.qop + (int64_t)b * kQOpWords * 64, lane);
  const SampleGeom sg = sample_geom(L, kDecCap);
  float tau = A.force_tau ? A.tau_value : -INFINITY;
  if (!A.force_tau && sg.n > 0) {
    const KeyBuf kbuf = make_keybuf(A.k, A.k_scale, (int64_t)A.num_pages * 64);
    const TilePaged tm{pt};
    const auto key_of = [&](int i) { return key_index(tm, kSampleOffset + sg.stride * min(i, sg.n - 1)); };
    KeyTile cur;
    load_tile_gather(cur, kbuf, [&](int i) { return key_of(i); }, lane);
#pragma unroll 1
    for (int i0 = 0; i0 < sg.n; i0 += kTile) {
      KeyTile nxt;
      load_tile_gather(nxt, kbuf, [&](int i) { return key_of(i0 + kTile + i); }, lane);
      const float sc = tile_score(qo, cur);
      if (i0 + (int)lane < sg.n) s_samp[wave][i0 + lane] = f2key(sc);
      cur = nxt;
    }
    wave_sync();
    const SelResult sel = wave_radix_select(SrcLds{s_samp[wave]}, sg.n, sg.r, s_hist[wave], lane, false);
    tau = key2f(sel.prefix);
  }
  if (lane == 0) {
    A.tau[b] = tau;
    A.status[b] = 0;
  }
}

// Workgroup (g, b) scores chunk g of sequence b; wave w takes the chunk's
// tiles w, w+4, ...  Its page ids are loaded once (lane i holds the page of
// its i-th tile, 64 tiles per reload) and key tiles are loaded two ahead.
// Keys >= tau go to the wave's LDS stage (slots from ballot + popcount); a
// stage that fills up mid-walk reserves a range of the sequence's
// candidate list with one device atomic and is copied there; at the end
// the workgroup reserves one range for all four stages.
__global__ __launch_bounds__(kWG) void k_decode_split(DecodeArgs A) {
  __shared__ uint2 s_stage[kWaves][kDecStage];
  __shared__ uint32_t s_cnt[kWaves], s_base[kWaves];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x, b = blockIdx.y;
  if (A.status[b] != 0) return;
  const int L = A.seq_lens[b];
  const int32_t* pt = A.table + (int64_t)b * A.max_pages;
  const int chunk = (((L + A.G - 1) / A.G) + 63) & ~63;
  const int k0 = g * chunk, k1 = min(L, k0 + chunk);
  if (k0 >= k1) return;
  const float tau = A.tau[b];
  uint32_t* ckey = A.cand_key + (int64_t)b * kDecCap;
  int32_t* cidx = A.cand_idx + (int64_t)b * kDecCap;
  uint32_t staged = 0u;
  // copy this wave's stage to [base, base + staged) of the list; entries
  // past the capacity are dropped, and the sequence keeps the largest
  // dropped key and the lowest dropped position (for the certificate)
  const auto copy_out = [&](uint32_t base) {
    uint32_t dk = 0u, dp = 0xFFFFFFFFu;
    for (uint32_t i = lane; i < staged; i += 64) {
      const uint2 e = s_stage[wave][i];
      if (base + i < (uint32_t)kDecCap) {
        ckey[base + i] = e.x;
        cidx[base + i] = (int32_t)e.y;
      } else {
        dk = max(dk, f2key(__uint_as_float(e.x)));
        dp = min(dp, e.y);
      }
    }
    if (dk) {
      atomicMax(&A.drop[2 * b], dk);
      atomicMin(&A.drop[2 * b + 1], dp);
    }
  };
  const KeyBuf kbuf = make_keybuf(A.k, A.k_scale, (int64_t)A.num_pages * 64);
  const int tile0 = (k0 >> 6) + wave;
  const int nt = tile0 < ((k1 + 63) >> 6) ? (((k1 + 63) >> 6) - tile0 + kWaves - 1) / kWaves : 0;
  if (nt > 0) {
    // page of the wave's i-th tile (clamped to its last tile past the end)
    int pg_lane = 0, pg_group = -1;
    const auto page_of = [&](int i) {
      i = min(i, nt - 1);
      if ((i >> 6) != pg_group) {
        pg_group = i >> 6;
        const int ti = (pg_group << 6) + (int)lane;
        pg_lane = pt[tile0 + kWaves * min(ti, nt - 1)];
      }
      return __builtin_amdgcn_readlane(pg_lane, i & 63);
    };
    int base0 = page_of(0) << 6, base1 = page_of(1) << 6;
    KeyTile t0, t1;
    load_tile(t0, kbuf, base0, lane);
    load_tile(t1, kbuf, base1, lane);
    QOp qo;
    load_qop(qo, A.qop + (int64_t)b * kQOpWords * 64, lane);
#pragma unroll 1
    for (int i = 0; i < nt; ++i) {
      const int base2 = page_of(i + 2) << 6;
      KeyTile t2;
      load_tile(t2, kbuf, base2, lane);
      const float sc = tile_score(qo, t0);
      const int my = ((tile0 + kWaves * i) << 6) + (int)lane;
      const bool take = my < k1 && sc >= tau;
      const uint64_t ball = __ballot(take);
      if (ball) {
        const uint32_t n = (uint32_t)__popcll(ball);
        if (staged + n > (uint32_t)kDecStage) {
          wave_sync();
          uint32_t base = 0u;
          if (lane == 0) base = atomicAdd(&A.cnt[b], staged);
          copy_out((uint32_t)__builtin_amdgcn_readfirstlane((int)base));
          staged = 0u;
          wave_sync();
        }
        if (take) s_stage[wave][staged + rank_in(ball)] = make_uint2(__float_as_uint(sc), (uint32_t)my);
        staged += n;
      }
      t0 = t1;
      t1 = t2;
      base0 = base1;
      base1 = base2;
    }
  }
  if (lane == 0) s_cnt[wave] = staged;
  __syncthreads();
  if (tid == 0) {
    const uint32_t total = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
    uint32_t base = total ? atomicAdd(&A.cnt[b], total) : 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      s_base[w] = base;
      base += s_cnt[w];
    }
  }
  __syncthreads();
  copy_out(s_base[wave]);
}

// One workgroup per sequence, after every chunk is in: load the candidate
// list into registers (32 keys per thread), select the K largest (ties at
// the K-th score to the lowest logical positions) and emit their physical
// slots, or put the sequence on the failure list.  The certificate is the
// prefill one: at least K candidates kept, no dropped candidate above the
// smallest selected score theta, and where one equals theta, the tied
// positions taken all below the lowest dropped position.  Also counts the
// remapped and invalid sequences.
__global__ __launch_bounds__(kWG) void k_decode_select(DecodeArgs A) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int b = blockIdx.x;
  uint32_t* stats = stat_copy(A.ctrl, blockIdx.x);
  const int st = A.status[b];
  if (tid == 0) atomicAdd(&stats[kStRows], 1u);
  if (st != 0) {
    if (tid == 0) atomicAdd(&stats[st == 1 ? kStTrivial : kStBad], 1u);
    return;
  }
  const uint32_t n = min(A.cnt[b], (uint32_t)kDecCap);
  const uint32_t drop = A.drop[2 * b], first_drop = A.drop[2 * b + 1];
  const int kr = A.K;  // L > K on this path
  bool ok = n >= (uint32_t)kr;
  if (ok) {
    const uint32_t* ckey = A.cand_key + (int64_t)b * kDecCap;
    const int32_t* cidx = A.cand_idx + (int64_t)b * kDecCap;
    const RegLayout lay = block_list_layout(n, (uint32_t)tid);
    uint32_t key[kDecCap / kWG];
    int32_t id[kDecCap / kWG];
    constexpr int M = kDecCap / kWG;
    load_list_regs(key, id, ckey, cidx, n, lay, [](uint32_t x) { return f2key(__uint_as_float(x)); });
    const auto kf = [&](int j) { return key[j]; };
    const RangeSel sel = (n > (uint32_t)kr) ? range_select_regs<M>(kf, lay, kr, sh, tid)
                                           : RangeSel{1u, 0xFFFFFFFFu, kr, (int)n};
    const uint32_t idlo = tie_bound_regs(key, id, lay, sel, sh, tid);
    if (drop >= sel.lo) {
      const uint32_t theta = range_min_regs<M>(kf, lay, sel, sh, tid);
      ok = drop <= theta;
      if (drop == theta) {  // tied keys were dropped: the taken ones must precede them
        uint32_t mn = 0xFFFFFFFFu;  // smallest ~position taken at theta
#pragma unroll
        for (int j = 0; j < M; ++j)
          if ((uint32_t)j < lay.jmax && key[j] == theta && ~(uint32_t)id[j] >= idlo) mn = min(mn, ~(uint32_t)id[j]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
        if (lane == 0) sh.wsum[0][tid >> 6] = mn;
        __syncthreads();
        mn = min(min(sh.wsum[0][0], sh.wsum[0][1]), min(sh.wsum[0][2], sh.wsum[0][3]));
        __syncthreads();
        ok = ok && ~mn < first_drop;
      }
    }
    if (ok)
      emit_range_regs(key, id, lay, sel, idlo, kr, A.K, A.out + (int64_t)b * A.K,
                      IdPaged{A.table + (int64_t)b * A.max_pages}, sh, tid);
  }
  if (tid == 0) {
    if (ok) {
      atomicAdd(&stats[kStFast], 1u);
    } else {
      const uint32_t f = atomicAdd(&A.ctrl[kCtrlFail], 1u);
      A.fail_list[f] = b;
      atomicAdd(&stats[drop ? kStOver : kStUnder], 1u);
    }
  }
}

__global__ __launch_bounds__(kWG) void k_decode_repair(DecodeArgs A) {
  __shared__ SelShared sh;
  __shared__ uint8_t s_qprep[kWaves][kUTerms * kD];
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t n_fail = __atomic_load_n(&A.ctrl[kCtrlFail], __ATOMIC_RELAXED);
  uint32_t* scratch = A.scratch + (int64_t)blockIdx.x * A.max_pages * 64;
  uint32_t* stats = stat_copy(A.ctrl, blockIdx.x);
#pragma unroll 1
  for (uint32_t f = blockIdx.x; f < n_fail; f += gridDim.x) {
    const int b = A.fail_list[f];
    const int L = A.seq_lens[b];
    const int32_t* pt = A.table + (int64_t)b * A.max_pages;
    QOp qo;
    prepare_q(qo, A.q, A.q_scale, A.w, b, lane, s_qprep[tid >> 6], 0);
    repair_row(qo, make_keybuf(A.k, A.k_scale, (int64_t)A.num_pages * 64), TilePaged{pt}, IdPaged{pt}, 0, L,
               A.K, A.out + (int64_t)b * A.K, scratch, sh, tid);
    if (tid == 0) atomicAdd(&stats[kStRepaired], 1u);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ host

static inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DecodeLayout {
  size_t ctrl, tau, status, cnt, drop, fail, ckey, cidx, scratch, qop, total;
};

static DecodeLayout decode_layout(int32_t B, int32_t max_pages) {
  DecodeLayout L;
  size_t o = 0;
  const size_t b = (size_t)(B > 0 ? B : 0);
  L.ctrl = o; o = a256(o + 4 * kCtrlWords);
  L.tau = o; o = a256(o + 4 * b);
  L.status = o; o = a256(o + 4 * b);
  L.cnt = o; o = a256(o + 4 * b);
  L.drop = o; o = a256(o + 8 * b);
  L.fail = o; o = a256(o + 4 * b);
  L.ckey = o; o = a256(o + 4 * b * kDecCap);
  L.cidx = o; o = a256(o + 4 * b * kDecCap);
  L.scratch = o; o = a256(o + 4 * (size_t)repair_grid(B) * (size_t)max_pages * 64);
  L.qop = o; o = a256(o + 4 * b * kQOpWords * 64);
  L.total = o;
  return L;
}

static int decode_split_count(int32_t B, int32_t max_pages) {
  // about 1024 workgroups in flight, but at least 1024 keys per workgroup
  int g = B > 0 ? 1024 / B : 1;
  const int by_len = (max_pages * 64) / 1024;
  if (g > by_len) g = by_len;
  if (g < 1) g = 1;
  if (g > 1024) g = 1024;
  return g;
}

size_t decode_workspace_bytes(int32_t B, int32_t max_pages, int32_t page_size, int32_t K) {
  if (B < 0 || max_pages < 0 || page_size != 64 || K < 1 || K > kKmax) return 0;
  return decode_layout(B, max_pages).total;
}

int decode_paged(const uint8_t* q, const float* q_scale, const uint8_t* k_cache, const float* k_scale,
                 const float* w, const int32_t* page_table, const int32_t* seq_lens, int32_t B,
                 int32_t max_pages, int32_t page_size, int32_t num_pages, int32_t K, int32_t* out_idx,
                 void* workspace, size_t workspace_bytes, hipStream_t stream, const idx_topk_opts* opts) {
  if (B < 0 || max_pages < 0 || num_pages < 0 || K < 1 || K > kKmax) return IDX_EINVAL;
  if (page_size != 64) return IDX_EUNSUPPORTED;
  if ((int64_t)max_pages * 64 > 0x7fffffffLL || (int64_t)num_pages * 64 > 0x7fffffffLL) return IDX_EINVAL;
  if (B == 0) return IDX_OK;
  if (!q || !w || !page_table || !seq_lens || !out_idx) return IDX_EINVAL;
  if (num_pages > 0 && (!k_cache || !k_scale)) return IDX_EINVAL;
  if (((uintptr_t)q & 15u) || ((uintptr_t)k_cache & 15u)) return IDX_EINVAL;
  const DecodeLayout L = decode_layout(B, max_pages);
  if (!workspace || workspace_bytes < L.total) return IDX_EWORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return IDX_EINVAL;
  char* ws = static_cast<char*>(workspace);
  DecodeArgs A;
  memset(&A, 0, sizeof(A));
  A.q = q; A.q_scale = q_scale; A.k = k_cache; A.k_scale = k_scale; A.w = w;
  A.table = page_table; A.seq_lens = seq_lens;
  A.B = B; A.max_pages = max_pages; A.num_pages = num_pages; A.K = K;
  A.G = decode_split_count(B, max_pages);
  A.out = out_idx;
  A.ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
  A.tau = reinterpret_cast<float*>(ws + L.tau);
  A.status = reinterpret_cast<int32_t*>(ws + L.status);
  A.cnt = reinterpret_cast<uint32_t*>(ws + L.cnt);
  A.drop = reinterpret_cast<uint32_t*>(ws + L.drop);
  A.fail_list = reinterpret_cast<int32_t*>(ws + L.fail);
  A.cand_key = reinterpret_cast<uint32_t*>(ws + L.ckey);
  A.cand_idx = reinterpret_cast<int32_t*>(ws + L.cidx);
  A.scratch = reinterpret_cast<uint32_t*>(ws + L.scratch);
  A.qop = reinterpret_cast<uint32_t*>(ws + L.qop);
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (opts) {
    A.force_tau = opts->force_tau ? 1 : 0;
    A.tau_value = opts->tau_value;
    ev0 = static_cast<hipEvent_t>(opts->ev_main_start);
    ev1 = static_cast<hipEvent_t>(opts->ev_main_stop);
  }
  hipLaunchKernelGGL(k_decode_prep, dim3((B + kWaves - 1) / kWaves), dim3(kWG), 0, stream, A);
  if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return IDX_EHIP;
  hipLaunchKernelGGL(k_decode_split, dim3(A.G, B), dim3(kWG), 0, stream, A);
  if (ev1 && hipEventRecord(ev1, stream) != hipSuccess) return IDX_EHIP;
  hipLaunchKernelGGL(k_decode_select, dim3(B), dim3(kWG), 0, stream, A);
  hipLaunchKernelGGL(k_decode_repair, dim3(repair_grid(B)), dim3(kWG), 0, stream, A);
  return hipGetLastError() == hipSuccess ? IDX_OK : IDX_EHIP;
}

}  // namespace idxk
