// Paged decode path (contest report page (arXiv 2608.14560), "DSA TopK Indexer"): one FP8 query
// per sequence against its keys in a paged FP8 cache with per-token scales.
//
//   k_decode_score  G workgroups per sequence split its keys (KV-dimension
//                   parallelism, Fusing Indexer Scoring and Exact Top-k
//                   page, "10. The optimization target after fusion");
//                   each scores its chunk with the prefill MFMA tile code
//                   and writes the FP32 scores at the keys' logical
//                   positions into the workspace.  For batches of up to 256
//                   sequences it also takes the sequence's sampled threshold
//                   from a few whole pages and stores the keys at or above
//                   it as candidates, per wave.
//   k_topk_rows     one workgroup per sequence (idx_rows.hip): checks the
//                   sequence's page ids, then the exact top-K of those
//                   candidates when there are at least K of them and none
//                   was dropped (every other key scores below the
//                   threshold), else of the score row itself; ties at the
//                   K-th score go to the lowest logical positions, emitted
//                   as physical cache slots.  Sequences with seq_len <= K
//                   take the remap path there (every slot, no selection).
//                   Larger batches pre-gather each score row above a cut
//                   sampled from the row itself (k_rows_gather) instead.
//
// The score row costs 4 bytes of writes per key against the 132 bytes of
// reads (codes and scale) that scoring needs anyway; it serves the exact
// fallback and the debug entry.  No host synchronisation anywhere.
#include <hip/hip_ext.h>
#include <string.h>

#include <mutex>

#include "idx_decode.hpp"
#include "idx_internal.hpp"
#include "idx_rows.hpp"

namespace idxk {

struct DecodeArgs {
  const uint8_t* q;
  const float* q_scale;
  const uint8_t* k;      // [num_pages*64][128]
  const float* k_scale;  // [num_pages*64]
  const float* w;
  const int32_t* table;  // [B][max_pages]
  const int32_t* seq_lens;
  int32_t B, max_pages, num_pages, K;
  int32_t G;             // fixed assignment: workgroups per sequence
  int32_t W;             // workgroups of the launch
  int32_t balanced;      // 1: workgroups assigned to sequences in proportion to their tiles
  uint32_t* ctrl;
  float* scores;         // [B][max_pages*64] scores at logical positions
  // filtered candidates (balanced assignment only; null otherwise): wave v
  // of workgroup g, the i-th of sequence b's, stores (order-preserving key,
  // logical position) pairs of its keys at or above the sequence's sampled
  // threshold into cand[(4g + v) * seg_cap ...] and their number (stored or
  // not) into cnt[b * kDecodeCntStride + 4i + v]; the first workgroup of
  // sequence b records plan[b] = (g, the sequence's workgroup count)
  uint2* cand;
  uint32_t* cnt;
  uint2* plan;
  int32_t seg_cap;
};

// One page of 64 keys (codes and scales) through buffer resources of its
// own, with a 64-bit base: a cache of any size is addressed, and a page id
// out of [0, num_pages) (or -1, a tile past a wave's share) gets empty
// resources, whose loads return zeros without a memory access.
__device__ __forceinline__ void load_page(KeyTile& t, const uint8_t* k, const float* k_scale, int num_pages, int pg,
                                          uint32_t lane) {
  const bool ok = pg >= 0 && pg < num_pages;
  const int64_t key0 = ok ? (int64_t)pg * 64 : 0;
  const rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + key0 * kD), (short)0, ok ? 64 * kD : 0, 0x00020000);
  const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(k_scale + key0), (short)0, ok ? 64 * 4 : 0, 0x00020000);
  const int voff = (int)(lane & 15) * kD + 32 * (int)(lane >> 4);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int soff = sub_off(c) * kD;
    const v4i x = __builtin_amdgcn_raw_buffer_load_b128(rk, voff, soff, 0);
    const v4i y = __builtin_amdgcn_raw_buffer_load_b128(rk, voff + 16, soff, 0);
    t.kb[c] = cat8(x, y);
  }
  t.ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)lane * 4, 0, 0));
}

// Sampled threshold of a sequence ("3.2 Sampled threshold", Fusing Indexer
// Scoring and Exact Top-k page, applied per decode sequence), at that
// section's rate of about one key in 200 but taken as whole pages of the
// cache (64 keys each, read like any other tile) at a fixed stride over the
// sequence's full pages: P = ceil(ceil((L - 100) / 200) / 64) pages, at
// most kDecodeSamplePages, page j being logical page floor((2j+1) F / (2P))
// of the F = floor(L / 64) full ones.  tau is taken at the r-th largest of
// the 64 P sampled scores, r = ceil(64 P * kSampleTarget / L), so that about
// kSampleTarget keys are expected at or above it.  Sequences of at most
// kDecodeKeepAll keys keep every key.
constexpr int kDecodeSamplePages = 8;
constexpr int kDecodeKeepAll = 4096;
struct DecodeSample {
  int pages, full, r;  // sampled pages (0: keep every key), full pages, rank
};
__device__ __forceinline__ DecodeSample decode_sample(int L) {
  DecodeSample d{0, L >> 6, 0};
  if (L <= kDecodeKeepAll) return d;
  const int ns = (L - kSampleOffset + kSampleStride - 1) / kSampleStride;
  d.pages = min(kDecodeSamplePages, max(1, (ns + 63) >> 6));
  const int64_t n = 64 * (int64_t)d.pages;
  const int64_t r = (n * kSampleTarget + L - 1) / L;
  d.r = (int)(r < 1 ? 1 : (r > n ? n : r));
  return d;
}

// A threshold at or below the r-th largest of n <= 512 order-preserving
// score keys (keys[0..n) in LDS, all nonzero), found by one wave on its own
// with no barrier: the samples' score range [min, max] cut into 256 equal
// bins (monotone in the key), one histogram in the wave's own 256 LDS
// words, the bin holding the r-th largest found from the top, and the
// smallest sample in that bin returned.  1 <= r <= n.
__device__ __forceinline__ uint32_t wave_cut_bins(const uint32_t* keys, int n, int r, uint32_t lane, uint32_t* hist) {
  uint32_t k[8];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = (int)lane + 64 * j;
    k[j] = i < n ? keys[i] : 0u;  // 0: no sample
    mn = min(mn, k[j] ? k[j] : 0xFFFFFFFFu);
    mx = max(mx, k[j]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) hist[lane + 64 * q] = 0u;
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (mn == mx) return mn;  // every sample one value
  const float vlo = key2f(mn);
  const float scale = 256.0f / (key2f(mx) - vlo);
  const auto vbin = [&](uint32_t x) { return (uint32_t)fminf((key2f(x) - vlo) * scale, 255.0f); };
  wave_sync();
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (k[j]) atomicAdd(&hist[vbin(k[j])], 1u);
  wave_sync();
  uint32_t b, above, inb;
  wave_find_bucket(hist, r, lane, b, above, inb);
  uint32_t lo = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < 8; ++j) lo = (k[j] && vbin(k[j]) == b) ? min(lo, k[j]) : lo;
  return wave_min_u32(lo);
}

// Each workgroup scores one piece of one sequence: a run of its 64-key
// tiles (pages).  Balanced assignment (batches of at most 256 sequences):
// every workgroup computes the same plan from the lengths, a sequence with
// T tiles to score getting 1 + floor((W - B) T / sum T) workgroups (sum at
// most W), which split its tiles evenly, so that a long sequence no longer
// sets the kernel's time alone (equal lengths measured 16.6 us against
// 19.8 us for the same keys spread unevenly); larger batches take a fixed
// number of workgroups per sequence.  Sequences with nothing to score
// (L <= K: remapped; invalid lengths) get no workgroup; page ids are checked
// by the selection, and a bad one is harmless here (its page gets empty
// resources) and the sequence's scores are then discarded.  Wave w scores
// the piece's tiles w, w+4, ...: page ids are loaded once per 64 tiles
// (lane i holds the page of the wave's i-th tile) and key tiles two ahead.
// Lane l writes the score of key l of each tile (one coalesced 256-byte
// store per tile).  The prologue overlaps its round trips: the query's
// loads and the first page ids go out together, then the first two key
// tiles, and the query arithmetic runs while those are in flight (a page
// check or query preparation ahead of the first key load idled the memory
// system for about 4.5 us).
//
// With the balanced assignment the workgroup also filters: before its walk
// it takes the sequence's sampled threshold tau (every workgroup of the
// sequence samples the same pages, so all get the same tau: the four
// waves score the sampled pages into LDS, then each wave finds tau itself),
// and each wave stores the keys of its tiles that score at least tau as
// candidates into its own segment (slot = count + rank in the ballot; a
// segment holds seg_cap of them and counts the rest), so that the selection
// reads about 2K candidates per sequence instead of its whole score row.
__global__ __launch_bounds__(kWG, 2) void k_decode_score(DecodeArgs A) {
  __shared__ uint8_t s_qprep[kWaves][kUTerms * kD];
  __shared__ SelShared sh;
  __shared__ uint32_t s_samp[64 * kDecodeSamplePages];  // the sampled scores as order-preserving keys
  __shared__ uint32_t s_cut[kWaves][256];              // each wave's threshold histogram
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x;
  if (wg == 0) clear_ctrl(A.ctrl, tid);  // first kernel of the call
  int b = 0, p0 = 0, p1 = 0;              // this workgroup's piece: tiles [p0, p1) of sequence b
  int gi = -1;                            // its index among the sequence's workgroups (balanced)
  if (A.balanced) {
    int T = 0;
    if (tid < A.B) {
      const int L = A.seq_lens[tid];
      T = (L > A.K && L <= A.max_pages * 64) ? (L + 63) >> 6 : 0;
    }
    uint32_t Tsum, Gsum;
    block_exclusive_scan((uint32_t)T, sh, tid, Tsum);
    const int G = T > 0 ? 1 + (int)((int64_t)(A.W - A.B) * T / (int64_t)(Tsum > 0u ? Tsum : 1u)) : 0;
    const uint32_t first = block_exclusive_scan((uint32_t)G, sh, tid, Gsum);
    if (tid == 0) sh.bucket = 0xFFFFFFFFu;
    __syncthreads();
    if (G > 0 && (uint32_t)wg >= first && (uint32_t)wg < first + (uint32_t)G) {
      sh.bucket = (uint32_t)tid;
      sh.above = (uint32_t)wg - first;
      sh.inbucket = (uint32_t)G;
      sh.pad0 = (uint32_t)T;
    }
    __syncthreads();
    if (sh.bucket != 0xFFFFFFFFu) {
      b = (int)sh.bucket;
      const int64_t g = sh.above, Gb = sh.inbucket, Tb = sh.pad0;
      p0 = (int)(Tb * g / Gb);
      p1 = (int)(Tb * (g + 1) / Gb);
      gi = (int)g;
      if (g == 0 && tid == 0 && A.plan) A.plan[b] = make_uint2((uint32_t)wg, (uint32_t)Gb);
    }
  } else {
    b = wg / A.G;
    const int g = wg % A.G;
    const int L = A.seq_lens[b];
    if (L > A.K && L <= A.max_pages * 64) {
      const int chunk = (((L + A.G - 1) / A.G) + 63) & ~63;
      const int k0 = g * chunk;
      if (k0 < L) {
        p0 = k0 >> 6;
        p1 = (min(L, k0 + chunk) + 63) >> 6;
      }
    }
  }
  const bool filter = A.cand != nullptr;
  uint32_t ncand = 0u;  // this wave's candidates (wave-uniform)
  if (p0 < p1) {
    const int L = A.seq_lens[b];
    const int k1 = min(L, p1 << 6);  // the piece's last key + 1
    const int32_t* pt = A.table + (int64_t)b * A.max_pages;
    const int tile0 = p0 + wave;
    const int nt = tile0 < p1 ? (p1 - tile0 + kWaves - 1) / kWaves : 0;
    // scores through a buffer resource bounded by the piece's end: a store
    // past k1 (or of a padding step) is dropped by the bounds check, so no
    // store sits behind a branch; candidates likewise through the wave's
    // segment, bounded at seg_cap pairs
    const rsrc_t srow = __builtin_amdgcn_make_buffer_rsrc((void*)(A.scores + (int64_t)b * A.max_pages * 64),
                                                          (short)0, k1 * 4, 0x00020000);
    const rsrc_t crow = __builtin_amdgcn_make_buffer_rsrc(
        filter ? (void*)(A.cand + ((int64_t)wg * kWaves + wave) * A.seg_cap) : (void*)A.scores, (short)0,
        filter ? A.seg_cap * 8 : 0, 0x00020000);
    const DecodeSample ds = filter ? decode_sample(L) : DecodeSample{0, 0, 0};
    QRaw qr;
    prepare_q_load(qr, A.q, A.q_scale, A.w, b, lane);
    // Loads are issued unconditionally, with clamped indexes: a load behind a
    // branch makes every later wait a full drain (the memory counter retires
    // in order and the compiler cannot count a load it may have skipped).
    int ng = min(64, nt);
    int pg_lane = pt[max(0, tile0 + kWaves * min((int)lane, ng - 1))];
    // this wave's sample pages: j = wave and wave + 4 (a page id of -1, past
    // the sampled pages, reads nothing)
    int spg[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int sj = wave + 4 * j;
      const int lp = (int)((2 * (int64_t)sj + 1) * ds.full / (2 * max(ds.pages, 1)));
      const int id = pt[min(lp, max(ds.full - 1, 0))];
      spg[j] = sj < ds.pages ? id : -1;
    }
    // page of the group's i-th tile; past the group, -1: its loads return
    // zeros without a memory access, so the loop's last steps and the final
    // barrier do not wait out a round trip for tiles that are never used
    const auto page_of = [&](int i) { return i < ng ? __builtin_amdgcn_readlane(pg_lane, min(i, ng - 1)) : -1; };
    const auto load = [&](KeyTile& t, int i) { load_page(t, A.k, A.k_scale, A.num_pages, page_of(i), lane); };
    KeyTile ta, tb, tc, td;
    load(ta, 0);
    load(tb, 1);
    // both sample pages go out with the first two tiles, before the query
    // arithmetic
    load_page(tc, A.k, A.k_scale, A.num_pages, spg[0], lane);
    load_page(td, A.k, A.k_scale, A.num_pages, spg[1], lane);
    QOp qo;
    prepare_q_finish(qo, qr, lane, s_qprep[wave], 0);
    float tau = -INFINITY;  // keeps every key
    if (ds.pages > 0) {  // uniform over the workgroup
      const float sc0 = tile_score(qo, tc), sc1 = tile_score(qo, td);
      if (wave < ds.pages) s_samp[64 * wave + lane] = f2key(sc0);
      if (wave + 4 < ds.pages) s_samp[64 * (wave + 4) + lane] = f2key(sc1);
      __syncthreads();
      // every wave selects the threshold itself (the same value), with no
      // second barrier: the smallest sample in the bin of the r-th largest
      tau = key2f(wave_cut_bins(s_samp, 64 * ds.pages, ds.r, lane, s_cut[wave]));
    }
    // Groups of up to 64 of the wave's tiles.  Three tile buffers in
    // rotation give two tiles of lead; the roles rotate by unrolling rather
    // than by register copies, which would wait for the loads just issued
    // (the memory counter retires in order).  Within a group the loop
    // issues only tile loads and stores: a load behind a branch would make
    // every later wait a full drain.
#pragma unroll 1
    for (int g0 = 0; g0 < nt; g0 += 64) {
      if (g0 > 0) {  // the next group's page ids and first tiles (pieces of more than 16384 keys)
        ng = min(64, nt - g0);
        pg_lane = pt[tile0 + kWaves * (g0 + min((int)lane, ng - 1))];
        load(ta, 0);
        load(tb, 1);
      }
      const auto step = [&](KeyTile& use, KeyTile& refill, int i) {  // score tile i, load tile i + 2
        load(refill, i + 2);
        const float sc = tile_score(qo, use);
        const int my = ((tile0 + kWaves * (g0 + i)) << 6) + (int)lane;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), srow, i < ng ? my * 4 : 0x7FFFFFF0, 0, 0);
        if (filter) {
          const bool take = i < ng && my < k1 && sc >= tau;
          const uint64_t ball = __ballot(take);
          const int off = take ? (int)((ncand + rank_in(ball)) * 8u) : 0x7FFFFFF0;
          const v2i c = {(int)f2key(sc), my};
          __builtin_amdgcn_raw_buffer_store_b64(c, crow, off, 0, 0);
          ncand += (uint32_t)__popcll(ball);
        }
      };
#pragma unroll 1
      for (int i = 0; i < ng; i += 3) {
        step(ta, tc, i);
        step(tb, ta, i + 1);
        step(tc, tb, i + 2);
      }
    }
  }
  // every wave of a sequence's workgroups reports its count (zero for an
  // empty piece), so that a selection never reads a count of an earlier call
  if (filter && gi >= 0 && lane == 0) A.cnt[(int64_t)b * kDecodeCntStride + gi * kWaves + wave] = ncand;
}

// ------------------------------------------------------------------ host

static inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Pre-gather before the per-sequence selection: gather workgroups per
// sequence (a power of two, about 512 in all); each one's region holds
// what its threads of the selection kernel hold in registers, 6144 / split.
constexpr int kDecGatherKeys = 6144;

// Scoring workgroups of a balanced launch: two per CU, all resident at once.
constexpr int kDecodeWGs = 512;
static inline int decode_gather_split(int32_t B) {
  int g = 1;  // a power of two
  while (2 * g <= kMaxGatherSplit && 2 * g * B <= 512) g *= 2;
  return g;
}

struct DecodeLayout {
  size_t ctrl, scores, gcnt, gkey, gid, cand, cnt, plan, total;
  int32_t seg_cap;  // candidate pairs per scoring wave (balanced assignment)
};

static int decode_split_count(int32_t B, int32_t max_pages) {
  // about two workgroups per CU, but at least 1024 keys per workgroup
  int g = B > 0 ? 512 / B : 1;
  const int by_len = (max_pages * 64) / 1024;
  if (g > by_len) g = by_len;
  if (g < 1) g = 1;
  if (g > 1024) g = 1024;
  return g;
}

// Candidate segment of one scoring wave under the balanced assignment: a
// piece has at most ceil(B * max_pages / (W - B)) tiles (a sequence with T
// tiles gets more than (W - B) T / sum T workgroups), a wave a quarter of
// them, so the segment holds every key of its tiles, up to 8 B pairs kept
// within [512, 2048].  A wave expects about 2K / (4 G) candidates of a
// sequence with G workgroups, G being W / B on average, so 2 B per wave,
// and a sequence short enough to keep every key (4096) on one workgroup
// brings at most 1024 per wave; a wave that finds more than its segment
// holds is counted, and its sequence is selected from the score row
// instead.
static int32_t decode_seg_cap(int32_t B, int32_t max_pages) {
  const int64_t piece = ((int64_t)B * max_pages + (kDecodeWGs - B) - 1) / (kDecodeWGs - B) + 1;
  const int64_t cap = 64 * ((piece + kWaves - 1) / kWaves);
  const int64_t lim = 64 * ((8 * (int64_t)B + 63) / 64);
  const int64_t top = lim < 512 ? 512 : (lim > 2048 ? 2048 : lim);
  return (int32_t)(cap < top ? cap : top);
}

static DecodeLayout decode_layout(int32_t B, int32_t max_pages) {
  DecodeLayout L;
  size_t o = 0;
  const size_t b = (size_t)(B > 0 ? B : 0);
  const bool balanced = B <= kWG;
  L.ctrl = o; o = a256(o + 4 * kCtrlWords);
  L.scores = o; o = a256(o + 4 * b * (size_t)max_pages * 64);
  L.seg_cap = balanced ? decode_seg_cap(B, max_pages) : 0;
  if (balanced) {  // filtered candidates
    L.gcnt = L.gkey = L.gid = o;
    L.cand = o; o = a256(o + 8 * (size_t)kDecodeWGs * kWaves * (size_t)L.seg_cap);
    L.cnt = o; o = a256(o + 4 * b * (size_t)kDecodeCntStride);
    L.plan = o; o = a256(o + 8 * b);
  } else {  // pre-gather
    const size_t gs = (size_t)decode_gather_split(B);
    L.gcnt = o; o = a256(o + 4 * b * gs);
    L.gkey = o; o = a256(o + 4 * b * kDecGatherKeys);
    L.gid = o; o = a256(o + 4 * b * kDecGatherKeys);
    L.cand = L.cnt = L.plan = o;
  }
  L.total = o;
  return L;
}

size_t decode_workspace_bytes(int32_t B, int32_t max_pages, int32_t page_size, int32_t K) {
  if (B < 0 || max_pages < 0 || page_size != 64 || K < 1 || K > kKmax) return 0;
  return decode_layout(B, max_pages).total;
}

int decode_paged(const uint8_t* q, const float* q_scale, const uint8_t* k_cache, const float* k_scale,
                 const float* w, const int32_t* page_table, const int32_t* seq_lens, int32_t B,
                 int32_t max_pages, int32_t page_size, int32_t num_pages, int32_t K, int32_t* out_idx,
                 void* workspace, size_t workspace_bytes, hipStream_t stream, const idx_topk_opts* opts,
                 float* scores_out) {
  if (B < 0 || max_pages < 0 || num_pages < 0 || K < 1 || K > kKmax) return IDX_EINVAL;
  if (page_size != 64 || B > kMaxGridY) return IDX_EUNSUPPORTED;
  // slots and logical positions are int32; the cache itself may be of any size
  if ((int64_t)max_pages * 64 * 4 > 0x7fffffffLL || (int64_t)num_pages * 64 > 0x7fffffffLL) return IDX_EINVAL;
  if (opts && (opts->force_tau || opts->cand_cap || opts->row_status || opts->clock_out ||
               opts->math_only))
    return IDX_EINVAL;
  if (opts && (opts->main_reps < 0 || opts->main_reps > 1000)) return IDX_EINVAL;
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
  A.balanced = B <= kWG ? 1 : 0;  // the plan's scan covers one length per thread
  A.W = A.balanced ? kDecodeWGs : A.G * B;
  A.ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
  A.scores = reinterpret_cast<float*>(ws + L.scores);
  if (A.balanced) {  // the scoring kernel filters; the selection reads its candidates
    A.cand = reinterpret_cast<uint2*>(ws + L.cand);
    A.cnt = reinterpret_cast<uint32_t*>(ws + L.cnt);
    A.plan = reinterpret_cast<uint2*>(ws + L.plan);
    A.seg_cap = L.seg_cap;
  }
  hipEvent_t ev0 = opts ? static_cast<hipEvent_t>(opts->ev_main_start) : nullptr;
  hipEvent_t ev1 = opts ? static_cast<hipEvent_t>(opts->ev_main_stop) : nullptr;
  // the timing events, when given, are recorded by the launches themselves
  // (main_reps > 1 repeats the idempotent scoring kernel for timing)
  const int reps = opts && opts->main_reps > 1 ? opts->main_reps : 1;
  for (int r = 0; r < reps; ++r) {
    hipEvent_t e0 = r == 0 ? ev0 : nullptr, e1 = r == reps - 1 ? ev1 : nullptr;
    if (e0 || e1)
      hipExtLaunchKernelGGL(k_decode_score, dim3(A.W), dim3(kWG), 0, stream, e0, e1, 0, A);
    else
      hipLaunchKernelGGL(k_decode_score, dim3(A.W), dim3(kWG), 0, stream, A);
  }
  if (hipGetLastError() != hipSuccess) return IDX_EHIP;
  RowsArgs R{A.scores, (int64_t)max_pages * 64, nullptr, seq_lens, B, max_pages * 64, K, out_idx, A.ctrl,
             page_table, max_pages, num_pages,
             nullptr, nullptr, nullptr, 0, 0, nullptr, nullptr, nullptr, 0};
  int rc;
  if (A.balanced) {
    R.dcand = A.cand;
    R.dcnt = A.cnt;
    R.dplan = A.plan;
    R.dseg = A.seg_cap;
    rc = launch_topk_rows_filtered(R, stream);
  } else {
    R.gkey = reinterpret_cast<uint32_t*>(ws + L.gkey);
    R.gid = reinterpret_cast<int32_t*>(ws + L.gid);
    R.gcnt = reinterpret_cast<uint32_t*>(ws + L.gcnt);
    R.gsplit = decode_gather_split(B);
    R.gcap = kDecGatherKeys / R.gsplit;
    rc = launch_topk_rows_gathered(R, stream);
  }
  // the debug path hands out the score rows the selection read
  if (rc == IDX_OK && scores_out &&
      hipMemcpyAsync(scores_out, A.scores, sizeof(float) * (size_t)B * (size_t)max_pages * 64,
                     hipMemcpyDeviceToDevice, stream) != hipSuccess)
    rc = IDX_EHIP;
  return rc;
}

// ---------------------------------------------------- allocation-free call

// The allocation-free entry point's scratch: one array per GPU in the code
// object's device data, held until the process ends.  Its name is a
// host-side stand-in on the host; the device address of each GPU's copy is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[IDX_TOPK_NOALLOC_SCRATCH_BYTES];

static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

int decode_paged_noalloc(const uint8_t* q, const float* q_scale, const uint8_t* k_cache, const float* k_scale,
                         const float* w, const int32_t* page_table, const int32_t* seq_lens, int32_t B,
                         int32_t max_pages, int32_t page_size, int32_t num_pages, int32_t K, int32_t* out_idx,
                         hipStream_t stream) {
  const size_t need = decode_workspace_bytes(B, max_pages, page_size, K);
  if (need == 0 || B == 0)  // rejected arguments or an empty batch: the full call's checks answer, no HIP call
    return decode_paged(q, q_scale, k_cache, k_scale, w, page_table, seq_lens, B, max_pages, page_size, num_pages,
                        K, out_idx, nullptr, 0, stream, nullptr);
  if (need > IDX_TOPK_NOALLOC_SCRATCH_BYTES) return IDX_ESCRATCH;
  void* ws = scratch_address();
  if (!ws) return IDX_EHIP;
  return decode_paged(q, q_scale, k_cache, k_scale, w, page_table, seq_lens, B, max_pages, page_size, num_pages, K,
                      out_idx, ws, IDX_TOPK_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

}  // namespace idxk
