/*
 * idx_topk.h -- DSA Lightning Indexer scoring fused with exact per-row top-K
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation (Fusing Indexer Scoring and Exact Top-k page, "1.1 The problem" equation and
 * "2.3 Problem definition"):
 *
 *     I[t,s] = sum_{j<64} w[t,j] * ReLU( q[t,j] . k[s] )
 *
 * for every query row t and every key s in the row's half-open valid range
 * [row_start[t], row_end[t]), with q[t,j] = e4m3(q8[t,j,:]) * q_scale[t,j] and
 * k[s] = e4m3(k8[s,:]) * k_scale[s] (FP8 operands "each with scales"), and the
 * output is, per row, the K ids with the largest I, in no particular order.
 * The pages allow any valid id among equal scores (same section); this
 * library resolves a tie at the K-th score toward the lowest key ids (decode:
 * the lowest logical positions), on every path, so the selected set is a
 * function of the inputs (the order inside a row is not).  The result is
 * exact: a sampled threshold only decides whether the fast path's candidate
 * set certifies the answer ("3.2 Sampled threshold: turn maintenance into
 * filtering"); rows where it does not are recomputed by an exact repair
 * path.
 *
 * The paged decode variant follows the contest report page (arXiv 2608.14560), "DSA TopK
 * Indexer": one FP8 query per sequence, a paged FP8 key cache with per-token
 * FP32 scales, per-head weights and sequence lengths; sequences no longer
 * than K reduce to an index remap.
 *
 * Conventions for every entry point below:
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     keeps none of them after returning and allocates no device memory.
 *   - Scratch memory is the caller's `workspace` of at least the size
 *     returned by the matching *_workspace() query (256-byte aligned).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the default stream).  There is no host synchronisation.
 *   - Geometry is fixed: 64 heads, head dimension 128, 1 <= K <= 2048.
 *   - FP8 codes are OCP e4m3fn (max 448, no infinities); NaN codes are not
 *     allowed in the inputs.  Scales must be finite and > 0.
 *   - Argument errors detectable on the host return a negative IDX_E* code
 *     and enqueue nothing.  Ranges that can only be seen on the device
 *     (start > end, end > N, a page id outside the cache) make that row's
 *     output all -1 and count it in idx_topk_stats.bad_rows.
 *   - Output rows hold min(K, L) valid ids (L = the row's range length)
 *     followed by K - min(K, L) entries of -1.
 *   - Calls that share one workspace must not overlap in time.
 */
#ifndef IDX_TOPK_H
#define IDX_TOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IDX_TOPK_HEADS 64
#define IDX_TOPK_DIM 128
#define IDX_TOPK_KMAX 2048
#define IDX_TOPK_PAGE 64

/* Threshold sampler: keys row_start + OFFSET + STRIDE*i inside the row are
 * scored exactly; the threshold is the r-th largest sample score with
 * r = ceil(n_samples * TARGET / L), aiming at TARGET = 2K candidates
 * ("3.2 Sampled threshold": about 0.5% of the row, about twice K). */
#define IDX_TOPK_SAMPLE_STRIDE 200
#define IDX_TOPK_SAMPLE_OFFSET 100
#define IDX_TOPK_SAMPLE_TARGET 4096

enum {
  IDX_OK = 0,
  IDX_EINVAL = -1,       /* null pointer, negative size, bad alignment, K out of range */
  IDX_EUNSUPPORTED = -2, /* geometry the kernels do not implement (page_size != 64) */
  IDX_EWORKSPACE = -3,   /* workspace missing or smaller than the query returned */
  IDX_EHIP = -4,         /* a HIP launch or copy failed */
  IDX_ESCRATCH = -5      /* the call needs more scratch than the static array of
                            idx_topk_decode_paged_noalloc holds */
};

/* Per-call counters kept in the workspace (read with idx_topk_read_stats). */
typedef struct {
  uint32_t rows;       /* rows (or sequences) processed                         */
  uint32_t fast_ok;    /* rows certified by the sampled-threshold fast path     */
  uint32_t underflow;  /* fast path failed: fewer than K candidates             */
  uint32_t overflow;   /* fast path failed: a candidate dropped for lack of
                          capacity scores above the selection (or ties with
                          it below a selected tied id)                          */
  uint32_t many_cands; /* fast-path rows that kept more than 4096 candidates
                          (twice K at the default sampling target; informational) */
  uint32_t repaired;   /* rows recomputed by the exact repair path              */
  uint32_t trivial;    /* rows (sequences) with L <= K: no scoring needed       */
  uint32_t bad_rows;   /* rows with an invalid range or page id (output all -1) */
} idx_topk_stats;

/* Test and diagnosis knobs for idx_topk_prefill_debug (zero = default). */
typedef struct {
  int32_t force_tau;   /* 1: use tau_value as every row's threshold             */
  float tau_value;
  int32_t cand_cap;    /* >0: candidates the fast path stores per row (<= the
                          default 8192); a row with more fails its certificate
                          and is repaired (0: the default)                       */
  void *ev_main_start; /* hipEvent_t or NULL: recorded by the launch of the main  */
  void *ev_main_stop;  /*   scoring kernel at its start and at its end (timing only) */
  int32_t main_reps;   /* >1: the main scoring kernel is launched this many times
                          back to back (it is idempotent), ev_main_start with the
                          first launch and ev_main_stop with the last, so that a
                          small kernel's average duration is not dominated by
                          one dispatch (timing only; at most 1000)              */
  int32_t *row_status; /* prefill: [Q] int32 device array or NULL; receives each
                          row's outcome: IDX_ROW_FAST (certified by the fast
                          path), IDX_ROW_UNDERFLOW or IDX_ROW_OVERFLOW (the
                          certificate failed and the row was recomputed by the
                          exact repair path), IDX_ROW_BAD (invalid range)      */
  uint64_t *clock_out; /* prefill: [2] uint64 device array or NULL; the main
                          scoring kernel adds, over all its waves, the
                          shader-clock cycles ([0]) and the constant-rate
                          wall-clock ticks ([1]) each wave ran for, so that
                          [0]/[1] times the wall-clock rate is the kernel's mean
                          shader clock.  The caller zeroes it before the call.  */
  int32_t math_only;   /* prefill, 1: control build of the main kernel (timing
                          only): the same key loads, MFMAs and head-weighted
                          scores, folded into a per-row checksum instead of
                          being filtered; no candidates, no selection, no
                          repair.  out_idx, scores_out and tau_out are not
                          written.  Needs force_tau = 0.                       */
} idx_topk_opts;

/* Row outcomes written to idx_topk_opts.row_status. */
#define IDX_ROW_FAST 0
#define IDX_ROW_UNDERFLOW 1
#define IDX_ROW_OVERFLOW 2
#define IDX_ROW_BAD (-1)

/* Bytes of workspace idx_topk_prefill needs for Q rows over N keys. */
size_t idx_topk_prefill_workspace(int32_t Q, int32_t N, int32_t K);

/*
 * How the main kernel walks Q rows over N keys (diagnostic, host only, no GPU call): *shared = 1
 * for the shared walk (eight rows per workgroup, each key tile staged once in LDS for four row
 * pairs), 0 for the one-pair walk; *splits = workgroups each row's key tiles are split over;
 * *segments = candidate segments per row.  Any output pointer may be NULL.  Returns IDX_OK, or
 * IDX_EINVAL for Q < 0 or N < 0.
 */
int idx_topk_prefill_geometry(int32_t Q, int32_t N, int32_t* shared, int32_t* splits, int32_t* segments);

/*
 * Prefill: top-K ids per query row (Fusing Indexer Scoring and Exact Top-k page, "2.3 Problem
 * definition").
 *   q         [Q][64][128] uint8 e4m3fn codes, 16-byte aligned
 *   q_scale   [Q][64] float > 0, or NULL for all-ones
 *   k         [N][128] uint8 e4m3fn codes, 16-byte aligned; (N + 64)*128 must
 *             fit in 31 bits (IDX_EUNSUPPORTED otherwise)
 *   k_scale   [N] float > 0
 *   w         [Q][64] float head weights
 *   row_start [Q] int32, row_end [Q] int32: valid range [start, end), 0 <= start <= end <= N
 *   K         1..2048
 *   out_idx   [Q][K] int32: absolute key ids in [start, end), unsorted, -1 padded
 * Returns IDX_OK or a negative IDX_E* code.
 */
int idx_topk_prefill(const uint8_t *q, const float *q_scale, const uint8_t *k,
                     const float *k_scale, const float *w, const int32_t *row_start,
                     const int32_t *row_end, int32_t K, int32_t *out_idx, int32_t Q,
                     int32_t N, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Same as idx_topk_prefill, plus diagnostics for tests:
 *   scores_out [Q][N] float or NULL: the FP32 score of every valid (t, s), as
 *              used by the selection (entries outside a row's range are not
 *              written);
 *   tau_out    [Q] float or NULL: the threshold each row was filtered with;
 *   opts       NULL or knobs that force the threshold or shrink capacities so
 *              that the repair path runs.
 */
int idx_topk_prefill_debug(const uint8_t *q, const float *q_scale, const uint8_t *k,
                           const float *k_scale, const float *w, const int32_t *row_start,
                           const int32_t *row_end, int32_t K, int32_t *out_idx, int32_t Q,
                           int32_t N, void *workspace, size_t workspace_bytes, void *stream,
                           float *scores_out, float *tau_out, const idx_topk_opts *opts);

/* Bytes of workspace idx_topk_prefill_unfused needs: that of idx_topk_prefill
 * plus the [Q][N] FP32 score matrix (2 GiB at Q = 4096, N = 131072). */
size_t idx_topk_prefill_unfused_workspace(int32_t Q, int32_t N, int32_t K);

/*
 * Unfused comparator of idx_topk_prefill (Fusing Indexer Scoring and Exact Top-k page,
 * "2.2 Indexer scoring is compute-bound": a scoring kernel writes the full score matrix, a
 * separate top-k reads it back).  Same arguments and output as
 * idx_topk_prefill: the same MFMA scoring (bit-identical scores) writes all
 * valid scores of every row into the workspace, then idx_topk_rows' kernel
 * selects each row from that matrix.  With the lowest-id tie rule both paths
 * return the same id set per row.  opts may be NULL or carry only the timing
 * events (ev_main_* bracket the scoring kernel); the other knobs give
 * IDX_EINVAL.  N * 4 must fit in 31 bits (IDX_EUNSUPPORTED otherwise).
 */
int idx_topk_prefill_unfused(const uint8_t *q, const float *q_scale, const uint8_t *k,
                             const float *k_scale, const float *w, const int32_t *row_start,
                             const int32_t *row_end, int32_t K, int32_t *out_idx, int32_t Q,
                             int32_t N, void *workspace, size_t workspace_bytes, void *stream,
                             const idx_topk_opts *opts);

/*
 * Exact top-K of every row of a dense FP32 matrix (the standalone selection
 * stage of Fusing Indexer Scoring and Exact Top-k page, "3.5 Stage result", Table 2).
 *   scores    device, 16-byte aligned; row t's value at position s is
 *             scores[t * ld + s]; only [row_start[t], row_end[t]) is read;
 *             NaN-free
 *   ld        row stride in floats, >= N
 *   row_start, row_end [Q] int32 device: 0 <= start <= end <= N (a row that
 *             breaks this gets all -1)
 *   K         1..2048
 *   out_idx   [Q][K] int32 device: the positions of the K largest values,
 *             unsorted; ties at the K-th value go to the lowest positions;
 *             rows with L = end - start <= K get all L positions then -1.
 * Needs no workspace (LDS only); N * 4 must fit in 31 bits.  Asynchronous on
 * `stream`.  Returns IDX_OK or a negative IDX_E* code.
 */
int idx_topk_rows(const float *scores, int64_t ld, const int32_t *row_start,
                  const int32_t *row_end, int32_t K, int32_t *out_idx, int32_t Q, int32_t N,
                  void *stream);

/* Bytes of workspace idx_topk_scan_bf16 needs: the [B][N] FP32 score rows plus
 * the gather regions (about B*N*4 + B*48 KiB). */
size_t idx_topk_scan_bf16_workspace(int32_t B, int32_t N, int32_t K);

/*
 * BF16 stream scan (the page "Deleting the key transpose puts the DSA indexer scan on its
 * streaming floor"): B independent streams, each with its own unquantised keys; stream b scores
 * every key i in [0, lens[b]) against its 64-head query,
 *   I[b,i] = sum_{j<64} w[b,j] * ReLU( q[b,j] . k[b,i] )   (FP32 accumulation),
 * and keeps the K largest.
 *   q        [B][64][128] BF16 bit patterns (uint16), 16-byte aligned
 *   w        [B][64] float
 *   k        [B][N][128] BF16 bit patterns, 16-byte aligned; stream b's keys at
 *            k + b*N*128; (N + 64)*256 must fit in 31 bits (IDX_EUNSUPPORTED)
 *   lens     [B] int32 device, 0 <= lens[b] <= N (a stream outside gets all -1)
 *   B        at most 65535 (IDX_EUNSUPPORTED)
 *   K        1..2048
 *   out_idx  [B][K] int32: key positions, unsorted, ties at the K-th score to the
 *            lowest positions, -1 padded (streams with lens[b] <= K get all
 *            their positions)
 *   opts     NULL or timing only (ev_main_* and main_reps for the scoring kernel)
 * Inputs must be finite (BF16 infinities and NaNs are not scored meaningfully).
 * Asynchronous on `stream`; returns IDX_OK or a negative IDX_E* code.
 */
int idx_topk_scan_bf16(const uint16_t *q, const float *w, const uint16_t *k, const int32_t *lens,
                       int32_t B, int32_t N, int32_t K, int32_t *out_idx, void *workspace,
                       size_t workspace_bytes, void *stream, const idx_topk_opts *opts);

/* Tests and diagnosis: the device address, inside a workspace used by the last
 * idx_topk_scan_bf16 call with these B and N, of its [B][N] FP32 score rows
 * (stream b's scores of positions [0, lens[b]) at row b; other entries
 * unspecified).  NULL for a NULL workspace or negative sizes. */
const float *idx_topk_scan_bf16_scores(const void *workspace, int32_t B, int32_t N);

/*
 * The scan's streaming floor (same page, "stream only: read keys, write one score, no math"):
 * reads n_records records of 256 bytes from src (16-byte aligned) and writes one
 * float per record to dst[n_records].  A measurement reference, not part of the
 * method.  Asynchronous on `stream`.
 */
int idx_topk_stream_floor(const void *src, int64_t n_records, float *dst, void *stream);

/* Bytes of workspace idx_topk_decode_paged needs. */
size_t idx_topk_decode_workspace(int32_t B, int32_t max_pages, int32_t page_size, int32_t K);

/*
 * Paged decode (contest report page (arXiv 2608.14560), "DSA TopK Indexer"): one query per
 * sequence b, keys at logical positions i in [0, seq_lens[b]) stored in page
 * page_table[b][i / page_size], slot i % page_size.
 *   q          [B][64][128] uint8 e4m3fn, 16-byte aligned
 *   q_scale    [B][64] float > 0, or NULL for all-ones
 *   k_cache    [num_pages][page_size][128] uint8 e4m3fn, 16-byte aligned
 *   k_scale    [num_pages][page_size] float > 0
 *   w          [B][64] float
 *   page_table [B][max_pages] int32 physical page ids
 *   seq_lens   [B] int32 (device), 0 <= seq_len <= max_pages * page_size
 *   B          at most 65535 (IDX_EUNSUPPORTED)
 *   page_size  must be 64
 *   out_idx    [B][K] int32: physical cache slots page*page_size + slot of the
 *              selected keys, unsorted, -1 padded; ties at the K-th score go
 *              to the lowest logical positions.  Sequences with
 *              seq_len <= K take the remap path: all their slots, no scoring.
 *              A sequence whose length is out of range or whose used page
 *              ids are outside [0, num_pages) gets all -1 (bad_rows count).
 * The keys are scored into a [B][max_pages*page_size] FP32 row per sequence in
 * the workspace.  For batches of up to 256 sequences the scoring kernel also
 * takes each sequence's sampled threshold (sequences longer than 4096 keys:
 * up to 8 whole pages at a fixed stride, "3.2 Sampled threshold" of the
 * Fusing Indexer Scoring and Exact Top-k page) and keeps the keys at or
 * above it as candidates; the selection is exact either way: from the
 * candidates when there are at least K of them and none was dropped
 * (counted as fast_ok), else from the score row (counted as underflow or
 * overflow, then fast_ok or repaired).  Larger batches select from the score
 * rows.  No host synchronisation; nothing is copied to the host.
 */
int idx_topk_decode_paged(const uint8_t *q, const float *q_scale, const uint8_t *k_cache,
                          const float *k_scale, const float *w, const int32_t *page_table,
                          const int32_t *seq_lens, int32_t B, int32_t max_pages,
                          int32_t page_size, int32_t num_pages, int32_t K, int32_t *out_idx,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Same as idx_topk_decode_paged, plus diagnostics for tests:
 *   scores_out [B][max_pages*page_size] float device array or NULL: for every
 *              sequence that was scored (K < seq_len, valid length
 *              and page ids) the FP32 score of logical position i at
 *              [b][i] for i < seq_len, exactly the values its selection read;
 *              other entries are unspecified.
 *   opts       NULL or timing only: ev_main_start/ev_main_stop are recorded by
 *              the launch of the split scoring kernel at its start and at its
 *              end, main_reps repeats it.  The decode path has no threshold
 *              or capacity knobs (its threshold is always sampled): opts
 *              with force_tau, cand_cap, row_status, clock_out or math_only
 *              set gives IDX_EINVAL.
 */
int idx_topk_decode_paged_debug(const uint8_t *q, const float *q_scale, const uint8_t *k_cache,
                                const float *k_scale, const float *w, const int32_t *page_table,
                                const int32_t *seq_lens, int32_t B, int32_t max_pages,
                                int32_t page_size, int32_t num_pages, int32_t K, int32_t *out_idx,
                                void *workspace, size_t workspace_bytes, void *stream,
                                float *scores_out, const idx_topk_opts *opts);

/*
 * Paged decode without any allocation, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, kernels
 * and output as idx_topk_decode_paged, minus the workspace: the scratch is a
 * static device array of IDX_TOPK_NOALLOC_SCRATCH_BYTES per GPU, set up by
 * the first call on each device (make that first call outside a graph
 * capture) and held until the process ends.  A call whose scratch would
 * exceed it (idx_topk_decode_workspace(B, max_pages, page_size, K) bytes)
 * returns IDX_ESCRATCH and enqueues nothing; the other errors are those of
 * idx_topk_decode_paged.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (two streams, two threads) race and
 * must be serialised by the caller.  Nothing is allocated or freed.
 */
#define IDX_TOPK_NOALLOC_SCRATCH_BYTES (16u << 20)
int idx_topk_decode_paged_noalloc(const uint8_t *q, const float *q_scale, const uint8_t *k_cache,
                                  const float *k_scale, const float *w, const int32_t *page_table,
                                  const int32_t *seq_lens, int32_t B, int32_t max_pages,
                                  int32_t page_size, int32_t num_pages, int32_t K, int32_t *out_idx,
                                  void *stream);

/* Copy the counters of the last call that used `workspace` into *out.
 * Synchronises `stream`.  For tests and diagnosis, not for hot loops. */
int idx_topk_read_stats(const void *workspace, idx_topk_stats *out, void *stream);

/* Static description of an error code. */
const char *idx_topk_strerror(int code);

/*
 * Graph capture of the multi-kernel calls.  A call of this library is a
 * short chain of kernels (up to nine for prefill); at small shapes their
 * launches, not their work, set the time of a call.  Recording the chain
 * once into a HIP graph and replaying it costs one launch per replay.
 *
 *   idx_topk_graph_begin(stream)   starts recording on `stream` (thread-local
 *                                  capture mode; the legacy NULL stream cannot
 *                                  be captured: IDX_EINVAL)
 *   ... any of idx_topk_prefill, _prefill_debug (no timing events),
 *       _prefill_unfused, _rows, _decode_paged, _scan_bf16, _stream_floor
 *       on `stream`, in any number and order ...
 *   idx_topk_graph_end(stream, &g) stops recording and instantiates the graph;
 *                                  on failure (a capture that was invalidated,
 *                                  a call that failed) returns IDX_EHIP, *g =
 *                                  NULL, and the stream is no longer capturing
 *   idx_topk_graph_launch(g, s)    replays every recorded kernel on stream s
 *                                  (any stream, also the NULL stream), in order
 *   idx_topk_graph_destroy(g)      frees the graph (NULL is ignored)
 *
 * Every pointer and size is recorded by value: each replay reads the same
 * input buffers (so new data goes into them before a replay), writes the
 * same outputs and uses the same workspace.  Replays on one workspace must
 * not overlap.  While a capture is open the recorded calls must not allocate
 * (callers pass their output and workspace buffers), must not carry timing
 * events (opts->ev_main_*: the capture then fails at
 * idx_topk_graph_end), and idx_topk_read_stats (which synchronises) must not
 * be called.  The graph object is host memory owned by the caller until
 * idx_topk_graph_destroy; nothing recorded clears memory with a memset node
 * (the chains clear their counters with kernels).
 */
typedef struct idx_topk_graph_s *idx_topk_graph;

int idx_topk_graph_begin(void *stream);
int idx_topk_graph_end(void *stream, idx_topk_graph *graph);
int idx_topk_graph_launch(idx_topk_graph graph, void *stream);
int idx_topk_graph_destroy(idx_topk_graph graph);

#ifdef __cplusplus
}
#endif

#endif /* IDX_TOPK_H */
