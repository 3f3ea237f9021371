/*
 * CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct reference for the DSA Lightning Indexer with
 * exact per-row top-K.  Only tests/, the smoke check in __graft_entry__.py and
 * the cpu_baseline leg of bench.py may load this library.  It shares no code
 * with the GPU library (scoring_exact_top_amd/csrc) and neither includes the
 * other.
 *
 * What it computes (Fusing Indexer Scoring and Exact Top-k page, "1.1 The problem" equation and
 * "2.3 Problem definition"):
 *
 *   I[t,s] = sum_{j<64} w[t,j] * ReLU( q[t,j] . k[s] ),     s in [start_t, end_t)
 *
 * with q[t,j] = dec(q8[t,j,:]) * q_scale[t,j] and k[s] = dec(k8[s,:]) * k_scale[s]
 * ("each with scales": the quantised operands are dequantised before the dot
 * product; q_scale may be absent, meaning 1).  dec() is the OCP FP8 e4m3fn
 * decode, built here from the bit fields.
 *
 * Every e4m3fn value is an integer multiple of 2^-9 with magnitude <= 448, so
 * each code product is an integer multiple of 2^-18 below 2^36 units and a
 * 128-term sum stays below 2^43 units: the raw dot product is EXACT in double
 * in any summation order.  Only the scale products, the ReLU-weighted head sum
 * and the final value round (relative ~1e-16).
 *
 * Selection: the whole valid row is sorted by (score descending, index
 * ascending); the first min(K, L) indices are the top-K, the rest of the
 * K output slots are -1.  The index tie-break only makes the oracle
 * deterministic: the pages allow any valid index among equal scores
 * ("2.3 Problem definition", exactness criterion).  theta is the K-th largest
 * score (the min(K,L)-th when L < K).
 *
 * -0 is canonicalised to +0 so that ordering on score values is total.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_H 64
#define OR_D 128

static double g_e4m3[256];
static int g_e4m3_ready = 0;

/* OCP FP8 e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m/8 * 2^-6 = m * 2^-9).  S.1111.111 is NaN;
 * there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448. */
static void e4m3_init(void) {
    if (g_e4m3_ready) return;
    for (int c = 0; c < 256; ++c) {
        int sign = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
        double v;
        if (e == 15 && m == 7)
            v = NAN;
        else if (e == 0)
            v = ldexp((double)m, -9);
        else
            v = ldexp(1.0 + (double)m / 8.0, e - 7);
        g_e4m3[c] = sign ? -v : v;
    }
    g_e4m3_ready = 1;
}

double oracle_e4m3_value(int code) {
    e4m3_init();
    return g_e4m3[code & 255];
}

/* Raw dot product of two 128-element code vectors, exact in double (see the
 * header).  Eight partial sums are used only for speed; exactness makes the
 * grouping immaterial. */
static double dot_raw_dec(const double *a, const double *b) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int d = 0; d < OR_D; d += 8)
        for (int i = 0; i < 8; ++i) acc[i] += a[d + i] * b[d + i];
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

double oracle_dot_raw(const uint8_t *a, const uint8_t *b) {
    e4m3_init();
    double x[OR_D], y[OR_D];
    for (int d = 0; d < OR_D; ++d) {
        x[d] = g_e4m3[a[d]];
        y[d] = g_e4m3[b[d]];
    }
    return dot_raw_dec(x, y);
}

/* One indexer score.  qd: the row's decoded codes [64][128]; qs: per-head q
 * scales (NULL = 1); w: head weights; kd: decoded key codes; ks: key scale. */
static double score_one(const double *qd, const float *qs, const float *w,
                        const double *kd, double ks) {
    double I = 0.0;
    for (int j = 0; j < OR_H; ++j) {
        double dot = dot_raw_dec(qd + (size_t)j * OR_D, kd);
        double x = (qs ? (double)qs[j] : 1.0) * ks * dot;   /* q[t,j] . k[s] */
        double relu = x > 0.0 ? x : 0.0;
        I += (double)w[j] * relu;
    }
    return I + 0.0; /* -0 -> +0 */
}

typedef struct {
    double v;
    int32_t i;
} sv_t;

static int cmp_desc(const void *pa, const void *pb) {
    const sv_t *a = (const sv_t *)pa, *b = (const sv_t *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

static int has_nan_row(const double *x, int n) {
    for (int i = 0; i < n; ++i)
        if (x[i] != x[i]) return 1;
    return 0;
}

/* Sort one row's scores and write top-K indices (remapped through idx_map
 * when given) and theta. */
static void select_row(sv_t *sv, int L, int K, const int32_t *idx_map, int32_t *out, double *theta) {
    qsort(sv, (size_t)L, sizeof(sv_t), cmp_desc);
    int kk = L < K ? L : K;
    for (int i = 0; i < K; ++i)
        out[i] = i < kk ? (idx_map ? idx_map[sv[i].i] : sv[i].i) : -1;
    if (theta) *theta = kk > 0 ? sv[kk - 1].v : NAN;
}

/*
 * Prefill oracle over a subset of rows.
 *   q [Q][64][128] codes, q_scale [Q][64] (or NULL), k [N][128] codes,
 *   k_scale [N], w [Q][64], row_start/row_end [Q] (half-open).
 *   rows[n_rows]: which rows to evaluate (NULL = 0..n_rows-1).
 *   scores_out [n_rows][N] double or NULL: the full row, NaN outside range.
 *   topk_out [n_rows][K]: absolute key ids, -1 padded.  theta_out [n_rows].
 * Returns 0, -1 on a bad argument or range, -2 on a NaN code in the input.
 */
int oracle_prefill_rows(const uint8_t *q, const float *q_scale, const uint8_t *k,
                        const float *k_scale, const float *w, const int32_t *row_start,
                        const int32_t *row_end, int32_t Q, int32_t N, int32_t K,
                        const int32_t *rows, int32_t n_rows, double *scores_out,
                        int32_t *topk_out, double *theta_out, int nthreads) {
    e4m3_init();
    if (!q || !k || !k_scale || !w || !row_start || !row_end || !topk_out || K < 1 || Q < 0 || N < 0)
        return -1;
    for (int r = 0; r < n_rows; ++r) {
        int t = rows ? rows[r] : r;
        if (t < 0 || t >= Q) return -1;
        if (row_start[t] < 0 || row_start[t] > row_end[t] || row_end[t] > N) return -1;
    }
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : err)
#endif
    {
        double *qd = (double *)malloc(sizeof(double) * OR_H * OR_D);
        double *kd = (double *)malloc(sizeof(double) * OR_D);
        sv_t *sv = (sv_t *)malloc(sizeof(sv_t) * (size_t)(N > 0 ? N : 1));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int r = 0; r < n_rows; ++r) {
            int t = rows ? rows[r] : r;
            const uint8_t *qrow = q + (size_t)t * OR_H * OR_D;
            for (int i = 0; i < OR_H * OR_D; ++i) qd[i] = g_e4m3[qrow[i]];
            if (has_nan_row(qd, OR_H * OR_D)) err |= 2;
            int s0 = row_start[t], s1 = row_end[t], L = s1 - s0;
            for (int s = s0; s < s1; ++s) {
                const uint8_t *krow = k + (size_t)s * OR_D;
                for (int d = 0; d < OR_D; ++d) kd[d] = g_e4m3[krow[d]];
                if (has_nan_row(kd, OR_D)) err |= 2;
                sv[s - s0].v = score_one(qd, q_scale ? q_scale + (size_t)t * OR_H : NULL,
                                         w + (size_t)t * OR_H, kd, (double)k_scale[s]);
                sv[s - s0].i = s;
            }
            if (scores_out) {
                double *so = scores_out + (size_t)r * N;
                for (int s = 0; s < N; ++s) so[s] = NAN;
                for (int i = 0; i < L; ++i) so[sv[i].i] = sv[i].v;
            }
            select_row(sv, L, K, NULL, topk_out + (size_t)r * K, theta_out ? theta_out + r : NULL);
        }
        free(qd);
        free(kd);
        free(sv);
    }
    return err ? -2 : 0;
}

/*
 * Paged decode oracle (contest report page (arXiv 2608.14560), "DSA TopK Indexer"): one query per
 * sequence b, logical positions i in [0, seq_lens[b]), key i lives in page
 * page_table[b][i / page_size] at slot i % page_size.  Output ids are physical
 * cache slots page * page_size + slot, -1 padded.
 *   q [B][64][128], q_scale [B][64] or NULL, k_cache [P][page_size][128],
 *   k_scale [P][page_size], w [B][64], page_table [B][max_pages], seq_lens [B].
 *   scores_out [B][max_len] or NULL: logical-position scores, NaN past seq_len.
 */
int oracle_decode(const uint8_t *q, const float *q_scale, const uint8_t *k_cache,
                  const float *k_scale, const float *w, const int32_t *page_table,
                  const int32_t *seq_lens, int32_t B, int32_t max_pages, int32_t page_size,
                  int32_t n_pages_total, int32_t K, double *scores_out, int32_t max_len,
                  int32_t *topk_out, double *theta_out, int nthreads) {
    e4m3_init();
    if (!q || !k_cache || !k_scale || !w || !page_table || !seq_lens || !topk_out || K < 1 ||
        page_size < 1 || B < 0)
        return -1;
    for (int b = 0; b < B; ++b) {
        int L = seq_lens[b];
        if (L < 0 || L > max_pages * page_size || (scores_out && L > max_len)) return -1;
        for (int p = 0; p < (L + page_size - 1) / page_size; ++p) {
            int pg = page_table[(size_t)b * max_pages + p];
            if (pg < 0 || pg >= n_pages_total) return -1;
        }
    }
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : err)
#endif
    {
        double *qd = (double *)malloc(sizeof(double) * OR_H * OR_D);
        double *kd = (double *)malloc(sizeof(double) * OR_D);
        int cap = max_pages * page_size;
        sv_t *sv = (sv_t *)malloc(sizeof(sv_t) * (size_t)(cap > 0 ? cap : 1));
        int32_t *phys = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap > 0 ? cap : 1));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int b = 0; b < B; ++b) {
            const uint8_t *qrow = q + (size_t)b * OR_H * OR_D;
            for (int i = 0; i < OR_H * OR_D; ++i) qd[i] = g_e4m3[qrow[i]];
            if (has_nan_row(qd, OR_H * OR_D)) err |= 2;
            int L = seq_lens[b];
            for (int i = 0; i < L; ++i) {
                int pg = page_table[(size_t)b * max_pages + i / page_size];
                int slot = pg * page_size + i % page_size;
                const uint8_t *krow = k_cache + (size_t)slot * OR_D;
                for (int d = 0; d < OR_D; ++d) kd[d] = g_e4m3[krow[d]];
                if (has_nan_row(kd, OR_D)) err |= 2;
                sv[i].v = score_one(qd, q_scale ? q_scale + (size_t)b * OR_H : NULL,
                                    w + (size_t)b * OR_H, kd, (double)k_scale[slot]);
                sv[i].i = i;
                phys[i] = slot;
            }
            if (scores_out) {
                double *so = scores_out + (size_t)b * max_len;
                for (int i = 0; i < max_len; ++i) so[i] = NAN;
                for (int i = 0; i < L; ++i) so[i] = sv[i].v;
            }
            select_row(sv, L, K, phys, topk_out + (size_t)b * K, theta_out ? theta_out + b : NULL);
        }
        free(qd);
        free(kd);
        free(sv);
        free(phys);
    }
    return err ? -2 : 0;
}

/* Exact top-K over an arbitrary score vector (used to select on the GPU's own
 * emitted scores for the bit-exact debug-path check).  Same ordering rule as
 * above; scores are taken as given (the caller canonicalises -0). */
int oracle_topk_of_scores(const double *scores, int32_t L, int32_t K, int32_t *out, double *theta) {
    if (!scores || !out || K < 1 || L < 0) return -1;
    sv_t *sv = (sv_t *)malloc(sizeof(sv_t) * (size_t)(L > 0 ? L : 1));
    for (int i = 0; i < L; ++i) {
        sv[i].v = scores[i] + 0.0;
        sv[i].i = i;
    }
    select_row(sv, L, K, NULL, out, theta);
    free(sv);
    return 0;
}

/*
 * BF16 stream scan oracle (the page "Deleting the key transpose puts the DSA indexer scan on its
 * streaming floor": every stream scores all of its own candidate keys, stored unquantised as
 * BF16, and keeps an exact top-2048).  Stream b has a BF16 query q[b][64][128],
 * head weights w[b][64] and keys k[b][i][128] for positions i in [0, lens[b]):
 *
 *   I[b,i] = sum_{j<64} w[b,j] * ReLU( q[b,j] . k[b,i] )
 *
 * BF16 is the upper half of an IEEE binary32: the value of the 16-bit pattern
 * x is the binary32 whose bits are x << 16.  A product of two BF16 values has
 * at most 16 significant bits, so it is exact in double; the 128-term sum and
 * the weighted head sum round at ~1e-16 relative.
 *   q [B][64][128], w [B][64], k [B][N][128] (16-bit patterns), lens [B].
 *   scores_out [B][N] double or NULL (NaN past lens[b]).
 *   topk_out [B][K]: positions, (score desc, index asc), -1 padded; theta_out [B].
 * Returns 0, -1 on a bad argument, -2 on a NaN or infinite input value.
 */
static double bf16_value(uint16_t x) {
    uint32_t u = (uint32_t)x << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_bf16_value(int bits) { return bf16_value((uint16_t)(bits & 0xFFFF)); }

int oracle_scan_bf16(const uint16_t *q, const float *w, const uint16_t *k, const int32_t *lens,
                     int32_t B, int32_t N, int32_t K, double *scores_out, int32_t *topk_out,
                     double *theta_out, int nthreads) {
    if (!q || !w || !k || !lens || !topk_out || K < 1 || B < 0 || N < 0) return -1;
    for (int b = 0; b < B; ++b)
        if (lens[b] < 0 || lens[b] > N) return -1;
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : err)
#endif
    {
        double *qd = (double *)malloc(sizeof(double) * OR_H * OR_D);
        double *kd = (double *)malloc(sizeof(double) * OR_D);
        sv_t *sv = (sv_t *)malloc(sizeof(sv_t) * (size_t)(N > 0 ? N : 1));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int b = 0; b < B; ++b) {
            const uint16_t *qrow = q + (size_t)b * OR_H * OR_D;
            for (int i = 0; i < OR_H * OR_D; ++i) qd[i] = bf16_value(qrow[i]);
            for (int i = 0; i < OR_H * OR_D; ++i)
                if (!isfinite(qd[i])) err |= 2;
            const float *wb = w + (size_t)b * OR_H;
            int L = lens[b];
            for (int s = 0; s < L; ++s) {
                const uint16_t *krow = k + ((size_t)b * N + s) * OR_D;
                for (int d = 0; d < OR_D; ++d) {
                    kd[d] = bf16_value(krow[d]);
                    if (!isfinite(kd[d])) err |= 2;
                }
                double I = 0.0;
                for (int j = 0; j < OR_H; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < OR_D; ++d) dot += qd[(size_t)j * OR_D + d] * kd[d];
                    I += (double)wb[j] * (dot > 0.0 ? dot : 0.0);
                }
                sv[s].v = I + 0.0;
                sv[s].i = s;
            }
            if (scores_out) {
                double *so = scores_out + (size_t)b * N;
                for (int s = 0; s < N; ++s) so[s] = NAN;
                for (int s = 0; s < L; ++s) so[s] = sv[s].v;
            }
            select_row(sv, L, K, NULL, topk_out + (size_t)b * K, theta_out ? theta_out + b : NULL);
        }
        free(qd);
        free(kd);
        free(sv);
    }
    return err ? -2 : 0;
}
