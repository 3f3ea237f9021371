"""Exactness checks against the oracle -- TEST INFRASTRUCTURE ONLY.

Criterion (Fusing Indexer Scoring and Exact Top-k page, "2.3 Problem definition"): every
returned id belongs to the row's half-open range, no id repeats, and the
multiset of scores of the returned ids is the multiset of the K largest
scores of the row; which of several equal-scoring ids is returned is free.
The GPU scores in FP32 and the oracle in fp64, so the selection is judged
with a relative tolerance REL_TOL around the oracle's K-th score theta, in
both directions:

  * every selected index s has I[s] >= theta - REL_TOL*|theta|
  * every index s with I[s] > theta + REL_TOL*|theta| is selected.

Scores emitted by the debug paths are judged element-wise:
  |S - I| <= REL_TOL*|I|   or   |S - I| <= GAMMA*B[s]
where B[s] = k_scale[s] * sum_j |w_j q_scale_j| * sum_d |dec(q)_jd dec(k)_sd| is the
magnitude that bounds FP32 rounding of the ~194-operation dot/ReLU/head sum
(standard forward error bound gamma_n = n*u/(1-n*u), n = 194, u = 2^-24).  The
second clause only matters where I itself cancels to near zero.  B is
computed by bound_from_values (both the FP8 and the BF16 paths use it).
"""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-3
GAMMA = 1.2e-5


class CheckError(AssertionError):
    pass


def _fail(msg):
    raise CheckError(msg)


def check_structure(out_row: np.ndarray, start: int, end: int, K: int, where: str = ""):
    """Exactly min(K, L) distinct ids in [start, end) followed by -1 padding."""
    L = end - start
    kk = min(K, L)
    out_row = np.asarray(out_row)
    if out_row.shape != (K,):
        _fail("%s: shape %s != (%d,)" % (where, out_row.shape, K))
    valid = out_row[:kk]
    pad = out_row[kk:]
    if np.any(pad != -1):
        _fail("%s: %d non -1 entries in the padding" % (where, int(np.sum(pad != -1))))
    if np.any(valid < start) or np.any(valid >= end):
        bad = valid[(valid < start) | (valid >= end)]
        _fail("%s: %d ids out of [%d,%d), e.g. %s" % (where, bad.size, start, end, bad[:5]))
    if np.unique(valid).size != kk:
        _fail("%s: duplicate ids (%d distinct of %d)" % (where, np.unique(valid).size, kk))


def check_selection(out_row, scores_row, start, end, K, theta, where="", rel_tol=REL_TOL):
    """Tolerance form of the exactness criterion, both directions.

    scores_row is indexed by absolute id (the oracle's full row).  Returns the
    number of selected ids whose exact score is below theta (ties broken the
    other way by rounding), for reporting.
    """
    check_structure(out_row, start, end, K, where)
    L = end - start
    kk = min(K, L)
    if kk == 0:
        return 0
    sel = np.asarray(out_row[:kk], dtype=np.int64)
    tol = rel_tol * abs(theta)
    sel_scores = scores_row[sel]
    low = sel_scores < theta - tol
    if np.any(low):
        _fail("%s: %d selected ids score below theta-tol (theta=%r, worst=%r)"
              % (where, int(low.sum()), theta, float(sel_scores.min())))
    mask = np.zeros(scores_row.shape[0], dtype=bool)
    mask[sel] = True
    rng = np.arange(start, end)
    above = rng[(scores_row[start:end] > theta + tol) & ~mask[start:end]]
    if above.size:
        _fail("%s: %d ids above theta+tol not selected (theta=%r, e.g. id %d score %r)"
              % (where, above.size, theta, int(above[0]), float(scores_row[above[0]])))
    return int(np.sum(sel_scores < theta))


def check_selection_rounding(out_row, scores_row, start, end, K, theta, bound_row, where="", gamma=GAMMA):
    """The selection judged at the scores' own rounding bound, for rows whose
    K-th score theta is so small against that bound that the relative bar
    of check_selection cannot be met in FP32 (theta near 0).  FP32 scoring
    can order two keys a, b against their exact scores only when
    |I[a] - I[b]| <= gamma*(B[a] + B[b]), the element-wise bound of
    check_scores.  With B_theta the largest bound among the ids scoring
    theta, every selected id s must have I[s] >= theta - gamma*(B[s] + B_theta)
    and every id s left out I[s] <= theta + gamma*(B[s] + B_theta).

    scores_row and bound_row are indexed by absolute id.  Returns the number
    of selected ids scoring below theta."""
    check_structure(out_row, start, end, K, where)
    kk = min(K, end - start)
    if kk == 0:
        return 0
    I = np.asarray(scores_row, dtype=np.float64)
    B = np.asarray(bound_row, dtype=np.float64)
    ids = np.arange(start, end)
    b_theta = float(np.max(B[ids[I[start:end] == theta]]))
    sel = np.asarray(out_row[:kk], dtype=np.int64)
    low = I[sel] < theta - gamma * (B[sel] + b_theta)
    if np.any(low):
        _fail("%s: %d selected ids below theta beyond the rounding bound (theta=%r, worst=%r)"
              % (where, int(low.sum()), theta, float(I[sel].min())))
    mask = np.zeros(I.shape[0], dtype=bool)
    mask[sel] = True
    out = ids[~mask[start:end]]
    high = I[out] > theta + gamma * (B[out] + b_theta)
    if np.any(high):
        _fail("%s: %d ids left out above theta beyond the rounding bound (theta=%r, e.g. id %d score %r)"
              % (where, int(high.sum()), theta, int(out[high][0]), float(I[out[high][0]])))
    return int(np.sum(I[sel] < theta))


def check_exact_values(out_row, scores_row, start, end, K, where=""):
    """Strict form of the pages' criterion on the oracle's own scores: the
    sorted selected scores equal the sorted true top-K scores exactly."""
    check_structure(out_row, start, end, K, where)
    kk = min(K, end - start)
    sel = np.sort(scores_row[np.asarray(out_row[:kk], dtype=np.int64)])
    true = np.sort(scores_row[start:end])[::-1][:kk][::-1]
    if not np.array_equal(sel, true):
        _fail("%s: sorted selected scores differ from the true top-K (%d mismatches)"
              % (where, int(np.sum(sel != true))))


def check_scores(S_gpu, I_oracle, bound=None, where="", rel_tol=REL_TOL, gamma=GAMMA):
    """Element-wise score tolerance.  Returns the count that passes only by the
    cancellation clause."""
    S = np.asarray(S_gpu, dtype=np.float64)
    I = np.asarray(I_oracle, dtype=np.float64)
    err = np.abs(S - I)
    ok_rel = err <= rel_tol * np.abs(I)
    if bound is None:
        ok = ok_rel
    else:
        ok = ok_rel | (err <= gamma * np.asarray(bound, dtype=np.float64))
    if not np.all(ok):
        i = int(np.argmax(~ok))
        _fail("%s: %d scores out of tolerance (e.g. #%d gpu=%r oracle=%r)"
              % (where, int((~ok).sum()), i, float(S.flat[i]), float(I.flat[i])))
    return int(np.sum(ok & ~ok_rel))


def check_debug_bitexact(out_row, S_row, start, end, K, where=""):
    """Selection on the GPU's own scores must be exact (bit for bit).

    S_row holds the GPU's FP32 scores indexed by absolute id.  theta_S is the
    K-th largest of S over the valid range.  Then: every id with S > theta_S is
    selected, the number selected at theta_S equals K - #(S > theta_S), and
    the sorted selected S values equal the sorted true top-K S values.
    """
    check_structure(out_row, start, end, K, where)
    kk = min(K, end - start)
    if kk == 0:
        return
    S = np.asarray(S_row, dtype=np.float32).astype(np.float64) + 0.0
    valid = S[start:end]
    order = np.sort(valid)[::-1]
    theta = order[kk - 1]
    sel = np.asarray(out_row[:kk], dtype=np.int64)
    sel_vals = S[sel]
    if not np.array_equal(np.sort(sel_vals)[::-1], order[:kk]):
        _fail("%s: selected GPU scores differ from the top-K of the GPU's own scores" % where)
    n_gt = int(np.sum(valid > theta))
    if int(np.sum(sel_vals > theta)) != n_gt:
        _fail("%s: not every id above theta_S selected" % where)
    if int(np.sum(sel_vals == theta)) != kk - n_gt:
        _fail("%s: wrong number taken at theta_S" % where)


def check_debug_canonical(out_row, S_row, start, end, K, where=""):
    """The library's tie rule on its own scores: the selected set is exactly
    {S > theta_S} plus the (K - #(S > theta_S)) lowest ids with S == theta_S,
    theta_S the K-th largest S in the valid range (-0 and +0 equal)."""
    check_structure(out_row, start, end, K, where)
    kk = min(K, end - start)
    if kk == 0:
        return
    S = np.asarray(S_row, dtype=np.float32).astype(np.float64) + 0.0
    ids = np.arange(start, end)
    valid = S[start:end]
    theta = np.sort(valid)[::-1][kk - 1]
    above = ids[valid > theta]
    tied = ids[valid == theta]          # ascending ids
    want = np.concatenate([above, tied[: kk - above.size]])
    got = np.sort(np.asarray(out_row[:kk], dtype=np.int64))
    if not np.array_equal(got, np.sort(want)):
        _fail("%s: selection differs from the lowest-id tie rule (%d ids differ)"
              % (where, int(np.setxor1d(got, want).size)))


def bound_from_values(qd, kd, wq, ks=None):
    """B[s] = ks[s] * sum_j |wq_j| * sum_d |qd[j,d]| * |kd[s,d]|  (numpy, fp64).

    qd [64, D] decoded query codes (no scale), kd [n, D] decoded key codes,
    wq [64] the head weights times the query scales, ks [n] key scales (None:
    all ones).  Every term is nonnegative, so B bounds |I| and the magnitude
    of every partial sum of the FP32 score computation."""
    qa = np.abs(np.asarray(qd, dtype=np.float64))           # [64, D]
    ka = np.abs(np.asarray(kd, dtype=np.float64))           # [n, D]
    per_head = ka @ qa.T                                     # [n, 64]: sum over d
    b = per_head @ np.abs(np.asarray(wq, dtype=np.float64))  # [n]: sum over heads
    return b if ks is None else np.asarray(ks, dtype=np.float64) * b


def score_bound(q8, q_scale, k8, k_scale, w, t, ids, e4m3_table):
    """B[t,s] of the FP8 path for row t and key ids `ids`."""
    ids = np.asarray(ids)
    qs = np.ones(64) if q_scale is None else q_scale[t].astype(np.float64)
    return bound_from_values(e4m3_table[q8[t]], e4m3_table[k8[ids]], w[t].astype(np.float64) * qs,
                             k_scale[ids].astype(np.float64))
