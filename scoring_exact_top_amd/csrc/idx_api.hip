// Host side of the C ABI declared in include/idx_topk.h: argument checks,
// workspace carving and kernel launches on the caller's stream.
#include <string.h>

#include "idx_internal.hpp"
#include "idx_decode.hpp"
#include "idx_rows.hpp"
#include "idx_scan.hpp"

namespace idxk {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct PrefillLayout {
  size_t ctrl, tau, fail, cand, segn, scratch, rhist, rrow, kt, dense, total;
};

// unfused: also the [Q][N] FP32 score matrix of the unfused comparator.
static PrefillLayout prefill_layout(int32_t Q, int32_t N, bool unfused = false) {
  PrefillLayout L;
  size_t o = 0;
  L.ctrl = o; o = align256(o + sizeof(uint32_t) * kCtrlWords);
  L.tau = o; o = align256(o + sizeof(float) * (size_t)Q);
  L.fail = o; o = align256(o + sizeof(int32_t) * (size_t)Q);
  const WalkGeom g = prefill_geom(Q, N);
  const size_t nseg = (size_t)g.nseg;
  const size_t cand = (size_t)Q * nseg * (size_t)prefill_seg_cap(g.nseg);
  L.cand = o; o = align256(o + sizeof(uint2) * cand);
  L.segn = o; o = align256(o + 4 * sizeof(uint32_t) * (size_t)Q * nseg);
  L.scratch = o; o = align256(o + sizeof(uint32_t) * (size_t)repair_rows(Q, N) * (size_t)repair_stride(N));
  L.rhist = o; o = align256(o + sizeof(uint32_t) * (size_t)repair_slots(Q, N) * kRepairDigits * 256);
  L.rrow = o; o = align256(o + sizeof(uint32_t) * (size_t)repair_slots(Q, N) * kRowWords);
  L.kt = o; o = align256(o + (size_t)((N + 63) / 64) * 64 * 128);
  L.dense = o; if (unfused) o = align256(o + sizeof(float) * (size_t)Q * (size_t)N);
  L.total = o;
  return L;
}

static int prefill_common(const uint8_t* q, const float* q_scale, const uint8_t* k,
                          const float* k_scale, const float* w, const int32_t* row_start,
                          const int32_t* row_end, int32_t K, int32_t* out_idx, int32_t Q, int32_t N,
                          void* workspace, size_t workspace_bytes, void* stream, float* scores_out,
                          float* tau_out, const idx_topk_opts* opts, bool unfused = false) {
  if (Q < 0 || N < 0 || K < 1 || K > kKmax) return IDX_EINVAL;
  if (Q == 0) return IDX_OK;
  if (!q || !w || !row_start || !row_end || !out_idx) return IDX_EINVAL;
  if (N > 0 && (!k || !k_scale)) return IDX_EINVAL;
  if (!aligned16(q) || (k && !aligned16(k))) return IDX_EINVAL;
  if (unfused && (int64_t)N * 4 > 0x7fffffffLL) return IDX_EUNSUPPORTED;
  // the relaid key tiles (and the key codes) are addressed with 31-bit offsets
  if (((int64_t)N + 64) * kD > 0x7fffffffLL) return IDX_EUNSUPPORTED;
  const PrefillLayout L = prefill_layout(Q, N, unfused);
  if (!workspace || workspace_bytes < L.total) return IDX_EWORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return IDX_EINVAL;
  char* ws = static_cast<char*>(workspace);

  PrefillArgs A;
  memset(&A, 0, sizeof(A));
  A.q = q; A.q_scale = q_scale; A.k = k; A.k_scale = k_scale; A.w = w;
  A.row_start = row_start; A.row_end = row_end;
  A.Q = Q; A.N = N; A.K = K;
  A.ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
  A.tau = reinterpret_cast<float*>(ws + L.tau);
  A.fail_list = reinterpret_cast<int32_t*>(ws + L.fail);
  A.cand = reinterpret_cast<uint2*>(ws + L.cand);
  A.segn = reinterpret_cast<uint32_t*>(ws + L.segn);
  const WalkGeom g = prefill_geom(Q, N);
  A.S = g.S;
  A.nseg = g.nseg;
  A.shared = g.shared;
  A.seg_cap = prefill_seg_cap(g.nseg);
  A.scratch = reinterpret_cast<uint32_t*>(ws + L.scratch);
  A.rhist = reinterpret_cast<uint32_t*>(ws + L.rhist);
  A.rrow = reinterpret_cast<uint32_t*>(ws + L.rrow);
  A.rslots = repair_slots(Q, N);
  A.rstride = repair_stride(N);
  A.kt = reinterpret_cast<uint8_t*>(ws + L.kt);
  A.out = out_idx;
  A.dbg_scores = scores_out;
  A.cand_cap = kCandCap;
  if (opts) {
    if (opts->cand_cap < 0 || opts->cand_cap > kCandCap) return IDX_EINVAL;
    if (opts->cand_cap > 0) A.cand_cap = opts->cand_cap;
    A.force_tau = opts->force_tau ? 1 : 0;
    A.tau_value = opts->tau_value;
    A.ev_main_start = static_cast<hipEvent_t>(opts->ev_main_start);
    A.ev_main_stop = static_cast<hipEvent_t>(opts->ev_main_stop);
    if (opts->main_reps < 0 || opts->main_reps > 1000) return IDX_EINVAL;
    A.main_reps = opts->main_reps;
    if (opts->math_only && (opts->force_tau || unfused)) return IDX_EINVAL;
    A.row_status = opts->row_status;
    A.clock = opts->clock_out;
    A.math_only = opts->math_only ? 1 : 0;
  }
  // usable entries per segment: the full segment unless a test knob shrank
  // the capacity, then an even share of it
  const int share = A.cand_cap / A.nseg;
  A.seg_eff = (A.cand_cap >= kCandCap || share > A.seg_cap) ? A.seg_cap : share;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (unfused) {
    A.dbg_scores = reinterpret_cast<float*>(ws + L.dense);
    A.force_tau = 1;
    A.tau_value = INFINITY;
    return launch_prefill_unfused(A, s);
  }
  // N <= kCandCap with the default capacities: every valid row has L <=
  // kCandCap, so its threshold is -inf, no segment overflows and the
  // certificate cannot fail (no sampling, no repair to launch)
  const bool small = !A.force_tau && A.N > 0 && A.N <= kCandCap && A.cand_cap >= kCandCap;
  A.keep_all = (small && !A.math_only) ? 1 : 0;
  // the one-pair walk of calls this short reads key tiles from k itself (the
  // control as the call it stands for); other calls read a relaid copy
  A.direct = (small && !A.shared) ? 1 : 0;
  // the main kernel samples its rows itself (with S > 1 splits per row pair,
  // each split samples the pair: the same values, S times, in parallel)
  A.fuse_tau = (!A.force_tau && !A.keep_all && !A.math_only && A.N > 0) ? 1 : 0;
  int rc = launch_prefill(A, s);
  if (rc == IDX_OK && tau_out) {
    if (hipMemcpyAsync(tau_out, A.tau, sizeof(float) * (size_t)Q, hipMemcpyDeviceToDevice, s) != hipSuccess)
      rc = IDX_EHIP;
  }
  return rc;
}

}  // namespace idxk

using namespace idxk;

extern "C" size_t idx_topk_prefill_workspace(int32_t Q, int32_t N, int32_t K) {
  if (Q < 0 || N < 0 || K < 1 || K > kKmax) return 0;
  return prefill_layout(Q, N).total;
}

extern "C" int idx_topk_prefill_geometry(int32_t Q, int32_t N, int32_t* shared, int32_t* splits,
                                         int32_t* segments) {
  if (Q < 0 || N < 0) return IDX_EINVAL;
  const WalkGeom g = prefill_geom(Q, N);
  if (shared) *shared = g.shared;
  if (splits) *splits = g.S;
  if (segments) *segments = g.nseg;
  return IDX_OK;
}

extern "C" int idx_topk_prefill(const uint8_t* q, const float* q_scale, const uint8_t* k,
                                const float* k_scale, const float* w, const int32_t* row_start,
                                const int32_t* row_end, int32_t K, int32_t* out_idx, int32_t Q,
                                int32_t N, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_common(q, q_scale, k, k_scale, w, row_start, row_end, K, out_idx, Q, N, workspace,
                        workspace_bytes, stream, nullptr, nullptr, nullptr);
}

extern "C" int idx_topk_prefill_debug(const uint8_t* q, const float* q_scale, const uint8_t* k,
                                      const float* k_scale, const float* w,
                                      const int32_t* row_start, const int32_t* row_end, int32_t K,
                                      int32_t* out_idx, int32_t Q, int32_t N, void* workspace,
                                      size_t workspace_bytes, void* stream, float* scores_out,
                                      float* tau_out, const idx_topk_opts* opts) {
  return prefill_common(q, q_scale, k, k_scale, w, row_start, row_end, K, out_idx, Q, N, workspace,
                        workspace_bytes, stream, scores_out, tau_out, opts);
}

extern "C" size_t idx_topk_prefill_unfused_workspace(int32_t Q, int32_t N, int32_t K) {
  if (Q < 0 || N < 0 || K < 1 || K > kKmax) return 0;
  return prefill_layout(Q, N, true).total;
}

extern "C" int idx_topk_prefill_unfused(const uint8_t* q, const float* q_scale, const uint8_t* k,
                                        const float* k_scale, const float* w, const int32_t* row_start,
                                        const int32_t* row_end, int32_t K, int32_t* out_idx, int32_t Q,
                                        int32_t N, void* workspace, size_t workspace_bytes, void* stream,
                                        const idx_topk_opts* opts) {
  if (opts && (opts->force_tau || opts->cand_cap || opts->row_status || opts->clock_out ||
               opts->math_only))
    return IDX_EINVAL;
  return prefill_common(q, q_scale, k, k_scale, w, row_start, row_end, K, out_idx, Q, N, workspace,
                        workspace_bytes, stream, nullptr, nullptr, opts, true);
}

extern "C" int idx_topk_rows(const float* scores, int64_t ld, const int32_t* row_start,
                             const int32_t* row_end, int32_t K, int32_t* out_idx, int32_t Q, int32_t N,
                             void* stream) {
  if (Q < 0 || N < 0 || K < 1 || K > kKmax) return IDX_EINVAL;
  if (Q == 0) return IDX_OK;
  if (!scores || !row_start || !row_end || !out_idx) return IDX_EINVAL;
  if (ld < N || ((uintptr_t)scores & 15u) != 0) return IDX_EINVAL;
  if ((int64_t)N * 4 > 0x7fffffffLL) return IDX_EUNSUPPORTED;
  RowsArgs R{scores, ld, row_start, row_end, Q, N, K, out_idx, nullptr};
  return launch_topk_rows(R, static_cast<hipStream_t>(stream));
}

extern "C" size_t idx_topk_scan_bf16_workspace(int32_t B, int32_t N, int32_t K) {
  return scan_bf16_workspace_bytes(B, N, K);
}

extern "C" int idx_topk_scan_bf16(const uint16_t* q, const float* w, const uint16_t* k, const int32_t* lens,
                                  int32_t B, int32_t N, int32_t K, int32_t* out_idx, void* workspace,
                                  size_t workspace_bytes, void* stream, const idx_topk_opts* opts) {
  return scan_bf16(q, w, k, lens, B, N, K, out_idx, workspace, workspace_bytes, static_cast<hipStream_t>(stream),
                   opts);
}

extern "C" const float* idx_topk_scan_bf16_scores(const void* workspace, int32_t B, int32_t N) {
  return scan_bf16_scores(workspace, B, N);
}

extern "C" int idx_topk_stream_floor(const void* src, int64_t n_records, float* dst, void* stream) {
  return stream_floor(src, n_records, dst, static_cast<hipStream_t>(stream));
}

extern "C" size_t idx_topk_decode_workspace(int32_t B, int32_t max_pages, int32_t page_size, int32_t K) {
  return decode_workspace_bytes(B, max_pages, page_size, K);
}

extern "C" int idx_topk_decode_paged(const uint8_t* q, const float* q_scale, const uint8_t* k_cache,
                                     const float* k_scale, const float* w, const int32_t* page_table,
                                     const int32_t* seq_lens, int32_t B, int32_t max_pages,
                                     int32_t page_size, int32_t num_pages, int32_t K, int32_t* out_idx,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_paged(q, q_scale, k_cache, k_scale, w, page_table, seq_lens, B, max_pages, page_size,
                      num_pages, K, out_idx, workspace, workspace_bytes, static_cast<hipStream_t>(stream), nullptr);
}

extern "C" int idx_topk_decode_paged_debug(const uint8_t* q, const float* q_scale, const uint8_t* k_cache,
                                           const float* k_scale, const float* w, const int32_t* page_table,
                                           const int32_t* seq_lens, int32_t B, int32_t max_pages,
                                           int32_t page_size, int32_t num_pages, int32_t K, int32_t* out_idx,
                                           void* workspace, size_t workspace_bytes, void* stream,
                                           float* scores_out, const idx_topk_opts* opts) {
  return decode_paged(q, q_scale, k_cache, k_scale, w, page_table, seq_lens, B, max_pages, page_size,
                      num_pages, K, out_idx, workspace, workspace_bytes, static_cast<hipStream_t>(stream), opts,
                      scores_out);
}

extern "C" int idx_topk_decode_paged_noalloc(const uint8_t* q, const float* q_scale, const uint8_t* k_cache,
                                             const float* k_scale, const float* w, const int32_t* page_table,
                                             const int32_t* seq_lens, int32_t B, int32_t max_pages,
                                             int32_t page_size, int32_t num_pages, int32_t K, int32_t* out_idx,
                                             void* stream) {
  return decode_paged_noalloc(q, q_scale, k_cache, k_scale, w, page_table, seq_lens, B, max_pages, page_size,
                              num_pages, K, out_idx, static_cast<hipStream_t>(stream));
}

extern "C" int idx_topk_read_stats(const void* workspace, idx_topk_stats* out, void* stream) {
  if (!workspace || !out) return IDX_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  static_assert(sizeof(idx_topk_stats) == sizeof(uint32_t) * kStatCount, "stats layout");
  const char* src = static_cast<const char*>(workspace) + sizeof(uint32_t) * kStatsOff;
  uint32_t copies[kStatLanes * kStatStride];
  if (hipMemcpyAsync(copies, src, sizeof(copies), hipMemcpyDeviceToHost, s) != hipSuccess) return IDX_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return IDX_EHIP;
  uint32_t sum[kStatCount] = {};
  for (int l = 0; l < kStatLanes; ++l)
    for (int c = 0; c < kStatCount; ++c) sum[c] += copies[l * kStatStride + c];
  memcpy(out, sum, sizeof(sum));
  return IDX_OK;
}

extern "C" const char* idx_topk_strerror(int code) {
  switch (code) {
    case IDX_OK: return "ok";
    case IDX_EINVAL: return "invalid argument";
    case IDX_EUNSUPPORTED: return "unsupported geometry";
    case IDX_EWORKSPACE: return "workspace missing or too small";
    case IDX_EHIP: return "HIP launch or copy failed";
    case IDX_ESCRATCH: return "call needs more scratch than the allocation-free entry point's static array";
    default: return "unknown error";
  }
}

// ---------------------------------------------------------------- graphs

struct idx_topk_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

extern "C" int idx_topk_graph_begin(void* stream) {
  if (!stream) return IDX_EINVAL;  // the legacy NULL stream cannot be captured
  return hipStreamBeginCapture(static_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal) == hipSuccess
             ? IDX_OK
             : IDX_EHIP;
}

extern "C" int idx_topk_graph_end(void* stream, idx_topk_graph* out) {
  if (out) *out = nullptr;
  if (!stream) return IDX_EINVAL;
  hipGraph_t g = nullptr;
  // ends the capture in every case, so that the stream is usable again
  if (hipStreamEndCapture(static_cast<hipStream_t>(stream), &g) != hipSuccess || !g) {
    (void)hipGetLastError();
    return IDX_EHIP;
  }
  if (!out) {
    (void)hipGraphDestroy(g);
    return IDX_EINVAL;
  }
  hipGraphExec_t e = nullptr;
  if (hipGraphInstantiate(&e, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return IDX_EHIP;
  }
  *out = new idx_topk_graph_s{g, e};
  return IDX_OK;
}

extern "C" int idx_topk_graph_launch(idx_topk_graph graph, void* stream) {
  if (!graph) return IDX_EINVAL;
  return hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)) == hipSuccess ? IDX_OK : IDX_EHIP;
}

extern "C" int idx_topk_graph_destroy(idx_topk_graph graph) {
  if (!graph) return IDX_OK;
  const bool ok = hipGraphExecDestroy(graph->exec) == hipSuccess && hipGraphDestroy(graph->graph) == hipSuccess;
  delete graph;
  return ok ? IDX_OK : IDX_EHIP;
}
