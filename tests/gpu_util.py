"""Helpers for GPU parity tests: move seeded cases to the device, run the
library through its C ABI binding, compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from oracle import check


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_prefill(case, device="cuda"):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(q8=t(case.q8), q_scale=None if case.q_scale is None else t(case.q_scale),
                k8=t(case.k8), k_scale=t(case.k_scale), w=t(case.w),
                row_start=t(case.row_start), row_end=t(case.row_end))


def run_prefill(case, debug=False, scores=False, status=False, **opts):
    import scoring_exact_top_amd as lib
    d = dev_prefill(case)
    ws = lib.alloc_workspace(lib.prefill_workspace_bytes(case.Q, case.N, case.K), "cuda")
    res = {}
    if debug or scores or status or opts:
        sc = torch.full((case.Q, case.N), float("nan"), dtype=torch.float32, device="cuda") if scores else None
        tau = torch.empty(case.Q, dtype=torch.float32, device="cuda")
        st = torch.full((case.Q,), -7, dtype=torch.int32, device="cuda") if status else None
        out = lib.prefill_debug(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                                d["row_end"], case.K, workspace=ws, scores_out=sc, tau_out=tau,
                                row_status=st, **opts)
        res["tau"] = tau.cpu().numpy()
        if scores:
            res["scores"] = sc.cpu().numpy()
        if status:
            res["status"] = st.cpu().numpy()
    else:
        out = lib.prefill(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                          d["row_end"], case.K, workspace=ws)
    torch.cuda.synchronize()
    res["out"] = out.cpu().numpy()
    res["stats"] = lib.read_stats(ws)
    return res


def check_prefill_rows(case, out, rows, nthreads=0, gpu_scores=None, e4m3=None):
    """Oracle check of the given rows: structure + tolerance selection, and,
    when the GPU's scores are given, element-wise score tolerance and the
    bit-exact selection on the GPU's own scores.  A row whose K-th score is
    too close to 0 for the relative selection bar (check_selection) is
    judged at the scores' rounding bound (check_selection_rounding), which
    needs the GPU's scores and the bound B; such rows are counted."""
    rows = np.asarray(rows, dtype=np.int32)
    topk, theta, sc = oracle.prefill_case(case, rows=rows, nthreads=nthreads)
    below = 0
    cancel = 0
    rounding = 0
    for j, t in enumerate(rows):
        s0, s1 = int(case.row_start[t]), int(case.row_end[t])
        where = "%s row %d" % (case.name, t)
        bound = None
        if gpu_scores is not None and s1 > s0:
            S = gpu_scores[t]
            ids = np.arange(s0, s1)
            bound = check.score_bound(case.q8, case.q_scale, case.k8, case.k_scale, case.w, t, ids,
                                      e4m3) if e4m3 is not None else None
            cancel += check.check_scores(S[s0:s1], sc[j][s0:s1], bound=bound, where=where)
            check.check_debug_bitexact(out[t], S, s0, s1, case.K, where=where)
            check.check_debug_canonical(out[t], S, s0, s1, case.K, where=where)
        try:
            below += check.check_selection(out[t], sc[j], s0, s1, case.K, theta[j], where=where)
        except check.CheckError as e:
            if bound is None:
                raise
            full = np.zeros(sc[j].shape[0])
            full[s0:s1] = bound
            below += check.check_selection_rounding(out[t], sc[j], s0, s1, case.K, theta[j], full, where=where)
            log("%s: judged at the rounding bound (%s)" % (where, e))
            rounding += 1
    return dict(rows=len(rows), below_theta=below, cancel_only=cancel, rounding_only=rounding)


def sample_rows(Q, n, seed=0):
    """First, last, middle and random rows."""
    rng = np.random.default_rng(seed)
    base = {0, Q - 1, Q // 2}
    extra = rng.choice(Q, size=min(Q, n), replace=False).tolist()
    return np.array(sorted(base | set(extra)))[: max(n, 3)]


def audit_rows(case, out, rows=None, batch=128, gpu_scores=None, e4m3=None):
    """check_prefill_rows over the given rows (default: every row), in
    batches so that the oracle's fp64 score rows stay a few hundred MB; the
    oracle runs on all host threads."""
    rows = np.arange(case.Q) if rows is None else np.asarray(rows)
    tot = dict(rows=0, below_theta=0, cancel_only=0, rounding_only=0)
    for i in range(0, rows.size, batch):
        rep = check_prefill_rows(case, out, rows[i:i + batch], gpu_scores=gpu_scores, e4m3=e4m3)
        for k in tot:
            tot[k] += rep[k]
    return tot


def status_matches_stats(status, stats):
    """Per-row outcomes agree with the call's counters."""
    import scoring_exact_top_amd as lib
    n_fast = int(np.sum(status == lib.ROW_FAST))
    n_under = int(np.sum(status == lib.ROW_UNDERFLOW))
    n_over = int(np.sum(status == lib.ROW_OVERFLOW))
    n_bad = int(np.sum(status == lib.ROW_BAD))
    assert n_fast + n_under + n_over + n_bad == status.size, "rows without an outcome"
    assert (n_fast, n_under, n_over, n_bad) == (stats["fast_ok"], stats["underflow"], stats["overflow"],
                                                stats["bad_rows"]), (n_fast, n_under, n_over, n_bad, stats)
    assert stats["repaired"] == n_under + n_over, stats
