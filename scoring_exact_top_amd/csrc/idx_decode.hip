// Paged decode path (contest report page (arXiv 2608.14560), "DSA TopK Indexer"): one FP8 query
// per sequence against its keys in a paged FP8 cache with per-token scales.
//
//   k_decode_score  G workgroups per sequence split its keys (KV-dimension
//                   parallelism, Fusing Indexer Scoring and Exact Top-k
//                   page, "10. The optimization target after fusion");
//                   each validates its pages, scores its chunk with the
//                   prefill MFMA tile code and writes the FP32 scores at
//                   the keys' logical positions into the workspace.
//   k_topk_rows     one workgroup per sequence (idx_rows.hip): exact top-K
//                   over the sequence's score row, ties at the K-th score to
//                   the lowest logical positions, emitted as physical cache
//                   slots.  Sequences with seq_len <= K take the remap path
//                   there (every slot, no selection).
//
// Unlike prefill, decode writes its scores out: a key costs 132 bytes of
// HBM reads (codes and scale) and its score 4 bytes of writes, so the score
// row adds 3% to the traffic, while a sampled threshold would need a
// separate sampling pass before the scoring (one sequence's sample is a
// chain of dependent gathers, about as long as the whole scoring kernel)
// and a certificate with a repair path.  No host synchronisation anywhere.
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
__global__ __launch_bounds__(kWG, 2) void k_decode_score(DecodeArgs A) {
  __shared__ uint8_t s_qprep[kWaves][kUTerms * kD];
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x;
  if (wg == 0) clear_ctrl(A.ctrl, tid);  // first kernel of the call
  int b = 0, p0 = 0, p1 = 0;              // this workgroup's piece: tiles [p0, p1) of sequence b
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
  if (p0 >= p1) return;
  const int k1 = min(A.seq_lens[b], p1 << 6);  // the piece's last key + 1
  const int32_t* pt = A.table + (int64_t)b * A.max_pages;
  const int tile0 = p0 + wave;
  const int nt = tile0 < p1 ? (p1 - tile0 + kWaves - 1) / kWaves : 0;
  if (nt == 0) return;
  {
    // scores through a buffer resource bounded by the piece's end: a store
    // past k1 (or of a padding step) is dropped by the bounds check, so no
    // store sits behind a branch
    const rsrc_t srow = __builtin_amdgcn_make_buffer_rsrc((void*)(A.scores + (int64_t)b * A.max_pages * 64),
                                                          (short)0, k1 * 4, 0x00020000);
    QRaw qr;
    prepare_q_load(qr, A.q, A.q_scale, A.w, b, lane);
    int ng = min(64, nt);
    int pg_lane = pt[tile0 + kWaves * min((int)lane, ng - 1)];
    // page of the group's i-th tile; past the group, -1: its loads return
    // zeros without a memory access, so the loop's last steps and the final
    // barrier do not wait out a round trip for tiles that are never used
    const auto page_of = [&](int i) { return i < ng ? __builtin_amdgcn_readlane(pg_lane, min(i, ng - 1)) : -1; };
    const auto load = [&](KeyTile& t, int i) { load_page(t, A.k, A.k_scale, A.num_pages, page_of(i), lane); };
    KeyTile ta, tb, tc;
    load(ta, 0);
    load(tb, 1);
    QOp qo;
    prepare_q_finish(qo, qr, lane, s_qprep[wave], 0);
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
      };
#pragma unroll 1
      for (int i = 0; i < ng; i += 3) {
        step(ta, tc, i);
        step(tb, ta, i + 1);
        step(tc, tb, i + 2);
      }
    }
  }
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
  size_t ctrl, scores, gcnt, gkey, gid, total;
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

static DecodeLayout decode_layout(int32_t B, int32_t max_pages) {
  DecodeLayout L;
  size_t o = 0;
  const size_t b = (size_t)(B > 0 ? B : 0);
  L.ctrl = o; o = a256(o + 4 * kCtrlWords);
  L.scores = o; o = a256(o + 4 * b * (size_t)max_pages * 64);
  const size_t gs = (size_t)decode_gather_split(B);
  L.gcnt = o; o = a256(o + 4 * b * gs);
  L.gkey = o; o = a256(o + 4 * b * kDecGatherKeys);
  L.gid = o; o = a256(o + 4 * b * kDecGatherKeys);
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
             reinterpret_cast<uint32_t*>(ws + L.gkey), reinterpret_cast<int32_t*>(ws + L.gid),
             reinterpret_cast<uint32_t*>(ws + L.gcnt), kDecGatherKeys / decode_gather_split(B),
             decode_gather_split(B)};
  int rc = launch_topk_rows_gathered(R, stream);
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
