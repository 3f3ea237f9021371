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


def run_prefill(case, debug=False, scores=False, **opts):
    import scoring_exact_top_amd as lib
    d = dev_prefill(case)
    ws = lib.alloc_workspace(lib.prefill_workspace_bytes(case.Q, case.N, case.K), "cuda")
    res = {}
    if debug or scores or opts:
        sc = torch.full((case.Q, case.N), float("nan"), dtype=torch.float32, device="cuda") if scores else None
        tau = torch.empty(case.Q, dtype=torch.float32, device="cuda")
        out = lib.prefill_debug(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                                d["row_end"], case.K, workspace=ws, scores_out=sc, tau_out=tau, **opts)
        res["tau"] = tau.cpu().numpy()
        if scores:
            res["scores"] = sc.cpu().numpy()
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
    bit-exact selection on the GPU's own scores."""
    rows = np.asarray(rows, dtype=np.int32)
    topk, theta, sc = oracle.prefill_case(case, rows=rows, nthreads=nthreads)
    below = 0
    cancel = 0
    for j, t in enumerate(rows):
        s0, s1 = int(case.row_start[t]), int(case.row_end[t])
        where = "%s row %d" % (case.name, t)
        below += check.check_selection(out[t], sc[j], s0, s1, case.K, theta[j], where=where)
        if gpu_scores is not None and s1 > s0:
            S = gpu_scores[t]
            ids = np.arange(s0, s1)
            bound = check.score_bound(case.q8, case.q_scale, case.k8, case.k_scale, case.w, t, ids,
                                      e4m3) if e4m3 is not None else None
            cancel += check.check_scores(S[s0:s1], sc[j][s0:s1], bound=bound, where=where)
            check.check_debug_bitexact(out[t], S, s0, s1, case.K, where=where)
            check.check_debug_canonical(out[t], S, s0, s1, case.K, where=where)
    return dict(rows=len(rows), below_theta=below, cancel_only=cancel)


def sample_rows(Q, n, seed=0):
    """First, last, middle and random rows."""
    rng = np.random.default_rng(seed)
    base = {0, Q - 1, Q // 2}
    extra = rng.choice(Q, size=min(Q, n), replace=False).tolist()
    return np.array(sorted(base | set(extra)))[: max(n, 3)]
