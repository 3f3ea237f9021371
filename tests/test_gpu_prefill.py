"""Prefill parity on MI355X: the HIP path through the C ABI against the CPU
oracle, element by element on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import check

pytestmark = pytest.mark.gpu

from gpu_util import check_prefill_rows, log, run_prefill, sample_rows, status_matches_stats  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import scoring_exact_top_amd  # noqa: F401  (fails loudly if the library is missing)


@pytest.fixture(scope="module")
def e4m3():
    return oracle.e4m3_table()


def test_small_ragged_all_rows_debug(e4m3):
    """Ragged random ranges (including empty and shorter-than-K rows) over
    several tiles with a tail; every row, plus scores and bit-exact check."""
    case = synth.random_case("ragged", 37, 5000, seed=21, K=1000, min_len=0)
    case.row_end[3] = case.row_start[3]          # an empty row
    log("case", case.name, case.Q, case.N)
    r = run_prefill(case, scores=True)
    rep = check_prefill_rows(case, r["out"], np.arange(case.Q), gpu_scores=r["scores"], e4m3=e4m3)
    log("ragged", rep, r["stats"])
    assert r["stats"]["rows"] == case.Q and r["stats"]["bad_rows"] == 0


@pytest.mark.parametrize("K", [1, 7, 64, 2048])
def test_k_values(K):
    case = synth.random_case("kvals", 9, 3000, seed=22 + K, K=K, min_len=0)
    log("K", K)
    r = run_prefill(case)
    check_prefill_rows(case, r["out"], np.arange(case.Q))


@pytest.mark.parametrize("name,Q,N,K,mode,opts", [
    ("one_row_short", 1, 100, 2048, "normal", {}),                # keeps every key, L < K
    ("keep_all_k17", 3, 8192, 17, "normal", {}),                  # keys read from k, 1024-thread select
    ("fused_257", 257, 8193, 2048, "normal", {}),                 # sampled threshold, 256-thread select
    ("fused_600", 600, 20000, 100, "normal", {}),
    ("repair_all", 64, 70000, 2048, "normal", {"force_tau": float("inf")}),
    ("repair_overflow", 40, 30000, 1000, "normal", {"force_tau": float("-inf"), "cand_cap": 600}),
    ("repair_ties", 5, 40000, 2048, "ties16", {"force_tau": float("inf")}),
])
def test_shape_sweep(name, Q, N, K, mode, opts):
    """Row counts on both sides of the select's workgroup-size switch (256
    rows), key counts on both sides of the keep-every-key bound (8192), K
    from 17 to 2048, and calls sent through the exact repair (underflow,
    overflow, a tie group in the gathered boundary group): ragged ranges,
    every row against the oracle."""
    if mode == "ties16":
        case = synth.causal_case(name, Q, N, seed=41, key_mode="ties16", K=K)
    else:
        case = synth.random_case(name, Q, N, seed=40 + Q, K=K, min_len=min(N, 50))
    log("case", name, Q, N, K, opts)
    r = run_prefill(case, **opts)
    st = r["stats"]
    log("stats", st)
    check_prefill_rows(case, r["out"], np.arange(case.Q))
    assert st["rows"] == case.Q and st["fast_ok"] + st["repaired"] == case.Q - st["bad_rows"], st
    if opts.get("force_tau") == float("inf"):
        long_rows = int(np.sum(case.row_end - case.row_start > K))
        assert st["repaired"] >= long_rows, st


def test_prefill_smoke_workload_full(e4m3):
    """64 rows at positions 8128..8191 of 8192 keys: every row, scores too."""
    case = synth.prefill_smoke(0)
    log("case", case.name)
    r = run_prefill(case, scores=True)
    rep = check_prefill_rows(case, r["out"], np.arange(case.Q), gpu_scores=r["scores"], e4m3=e4m3)
    log("smoke", rep, r["stats"])
    r2 = run_prefill(case)
    assert np.array_equal(np.sort(r2["out"], axis=1), np.sort(r["out"], axis=1))


def test_forced_underflow_goes_to_repair():
    case = synth.random_case("under", 12, 9000, seed=23, K=512, min_len=3000)
    log("case", case.name)
    r = run_prefill(case, force_tau=float("inf"))
    assert r["stats"]["underflow"] == case.Q and r["stats"]["repaired"] == case.Q
    check_prefill_rows(case, r["out"], np.arange(case.Q))


def test_forced_overflow_goes_to_repair():
    case = synth.random_case("over", 12, 9000, seed=24, K=512, min_len=3000)
    log("case", case.name)
    r = run_prefill(case, force_tau=float("-inf"), cand_cap=1024)
    assert r["stats"]["overflow"] == case.Q and r["stats"]["repaired"] == case.Q
    check_prefill_rows(case, r["out"], np.arange(case.Q))


def test_rows_keeping_every_key_merge_all_segments():
    """Rows that keep every key (threshold -inf, L <= 8192, the default
    capacity) hold more than 4096 candidates, spread over all their
    segments: the certificate holds for every row and the selection merges
    every segment.  Row 0 spans 8192 keys from an unaligned start, the most
    tiles one row can put on a segment."""
    case = synth.random_case("keep_all", 10, 9000, seed=25, K=700, min_len=4200, max_len=8192)
    case.row_start[0], case.row_end[0] = 1, 8193
    log("case", case.name)
    r = run_prefill(case, force_tau=float("-inf"), scores=True)
    st = r["stats"]
    log("stats", st)
    assert st["many_cands"] == case.Q and st["fast_ok"] == case.Q and st["repaired"] == 0, st
    check_prefill_rows(case, r["out"], np.arange(case.Q))


def _sample_tau(S_row, s0, s1):
    """The threshold the sampler must produce from the main kernel's own
    scores: r-th largest score at positions s0 + OFFSET + STRIDE*i inside the
    row (the sampling reading of the "3.2 Sampled threshold" section, as
    documented in include/idx_topk.h, for rows of at most 2048 samples)."""
    stride, offset, target = synth.SAMPLE_STRIDE, synth.SAMPLE_OFFSET, 4096
    L = s1 - s0
    n = -(-(L - offset) // stride)
    assert n <= 2048
    r = min(max(-(-(n * target) // L), 1), n)
    v = np.sort(S_row[s0 + offset + stride * np.arange(n)])[::-1]
    return v[r - 1]


def test_sampler_matches_main_scores_bit_for_bit(e4m3):
    """Even and odd rows (first and second row of a main-kernel pair) get the
    same scores from the sampler as from the main kernel, bit for bit, so a
    threshold equal to a sampled score keeps every copy of that score."""
    case = synth.random_case("sampled", 7, 24000, seed=28, K=2048, min_len=9000, max_len=24000)
    log("case", case.name)
    r = run_prefill(case, scores=True)
    for t in range(case.Q):
        s0, s1 = int(case.row_start[t]), int(case.row_end[t])
        want = np.float32(_sample_tau(r["scores"][t], s0, s1))
        assert r["tau"][t].view(np.uint32) == want.view(np.uint32), (t, r["tau"][t], want)
    check_prefill_rows(case, r["out"], np.arange(case.Q), gpu_scores=r["scores"], e4m3=e4m3)


def test_fused_sampler_bit_for_bit_with_ragged_ranges(e4m3):
    """1024 rows: one workgroup per row pair, so the main kernel samples its
    own rows.  Ragged ranges give the two rows of a pair different sample
    positions (a pass per row) or, for equal starts, shared ones; every
    threshold must be the r-th largest of the walk's own scores at the
    sampled positions, and sampled rows must match the oracle."""
    case = synth.random_case("fused_sampler", 1024, 20000, seed=29, K=2048, min_len=0, max_len=20000)
    case.row_start[1::4] = case.row_start[0::4]        # some pairs share their start
    case.row_end[1::4] = np.maximum(case.row_end[1::4], case.row_start[1::4])
    log("case", case.name)
    r = run_prefill(case, scores=True)
    for t in range(case.Q):
        s0, s1 = int(case.row_start[t]), int(case.row_end[t])
        if s1 - s0 <= 8192:
            assert r["tau"][t] == -np.inf, t
            continue
        want = np.float32(_sample_tau(r["scores"][t], s0, s1))
        assert r["tau"][t].view(np.uint32) == want.view(np.uint32), (t, r["tau"][t], want)
    check_prefill_rows(case, r["out"], np.arange(0, case.Q, 37), gpu_scores=r["scores"], e4m3=e4m3)


def test_shared_walk_bit_for_bit_with_the_pair_walk(e4m3):
    """4093 rows with ragged ranges take the shared walk (eight rows per
    workgroup, a pair per wave, each key tile staged once in LDS; 4093 is
    not a multiple of eight, so the last workgroup has a half pair and an
    absent one).  The first 64 rows alone take the one-pair walk.  Every row's scores must be
    the same bits on both walks, every threshold must be the walk's own
    sampled score, and sampled rows (the last ones among them) must match
    the oracle."""
    import dataclasses
    import scoring_exact_top_amd as lib
    assert lib.prefill_geometry(4093, 20000)[0] == 1 and lib.prefill_geometry(64, 20000)[0] == 0
    case = synth.random_case("shared_walk", 4093, 20000, seed=31, K=2048, min_len=0, max_len=20000)
    case.row_start[1::8] = case.row_start[0::8]        # some pairs share their start
    case.row_end[1::8] = np.maximum(case.row_end[1::8], case.row_start[1::8])
    log("case", case.name, case.Q, case.N)
    r = run_prefill(case, scores=True)
    n = 64
    sub = dataclasses.replace(case, name="shared_walk_head", q8=case.q8[:n], q_scale=case.q_scale[:n], w=case.w[:n],
                              row_start=case.row_start[:n], row_end=case.row_end[:n])
    r2 = run_prefill(sub, scores=True)
    assert np.array_equal(r["scores"][:n].view(np.uint32), r2["scores"].view(np.uint32))
    assert np.array_equal(r["tau"][:n].view(np.uint32), r2["tau"].view(np.uint32))
    for t in range(case.Q):
        s0, s1 = int(case.row_start[t]), int(case.row_end[t])
        if s1 - s0 <= 8192:
            assert r["tau"][t] == -np.inf, t
            continue
        want = np.float32(_sample_tau(r["scores"][t], s0, s1))
        assert r["tau"][t].view(np.uint32) == want.view(np.uint32), (t, r["tau"][t], want)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(case.Q - 11, case.Q), np.arange(0, case.Q, 97)]))
    rep = check_prefill_rows(case, r["out"], rows, gpu_scores=r["scores"], e4m3=e4m3)
    log("shared walk", rep, r["stats"])
    assert r["stats"]["rows"] == case.Q


@pytest.mark.parametrize("mode", ["keep_all", "overflow", "underflow"])
def test_shared_walk_edge_modes(mode, e4m3):
    """The shared walk (2048 rows, so two splits per group of eight rows)
    where every row keeps all its keys (N <= 8192: no sampling, no
    repair), where a shrunk capacity makes every row overflow, and where a
    threshold of +inf makes every row underflow; the last two go through
    the repair.  Every row against the oracle, with the GPU's scores (K =
    1024 of ragged rows puts some K-th scores near 0, where the selection is
    judged at the scores' rounding bound)."""
    import scoring_exact_top_amd as lib
    N = 6000 if mode == "keep_all" else 3000
    assert lib.prefill_geometry(2048, N) == (1, 2, 2)
    case = synth.random_case("shared_" + mode, 2048, N, seed=33, K=1024, min_len=0)
    opts = {}
    if mode == "overflow":
        opts = dict(force_tau=float("-inf"), cand_cap=512)
    elif mode == "underflow":
        opts = dict(force_tau=float("inf"))
    r = run_prefill(case, status=True, scores=True, **opts)
    st = r["stats"]
    rep = check_prefill_rows(case, r["out"], np.arange(case.Q), gpu_scores=r["scores"], e4m3=e4m3)
    log(mode, st, rep)
    status_matches_stats(r["status"], st)
    long_rows = int(np.sum(case.row_end - case.row_start > case.K))
    if mode == "keep_all":
        assert st["fast_ok"] == case.Q and st["repaired"] == 0
    elif mode == "overflow":
        assert st["overflow"] >= long_rows - 8 and st["repaired"] == st["overflow"] + st["underflow"]
    else:
        assert st["underflow"] >= long_rows


def test_massive_ties_take_the_fast_path(e4m3):
    """Rows over 16 distinct keys: the threshold is the top score, held by
    about 10K keys, far more than the segments hold (capacity cut to 4096).
    The dropped candidates all tie with the smallest selected score, so the
    certificate accepts every row without repair."""
    pos = np.arange(163840 - 8, 163840, dtype=np.int64)
    case = synth.causal_case("ties_fast", 8, 163840, seed=29, key_mode="ties16", positions=pos)
    log("case", case.name)
    r = run_prefill(case, scores=True, cand_cap=4096)
    st = r["stats"]
    log("stats", st)
    assert st["fast_ok"] == case.Q and st["repaired"] == 0, st
    check_prefill_rows(case, r["out"], np.arange(case.Q), gpu_scores=r["scores"], e4m3=e4m3)


def test_ties_through_repair_take_the_lowest_ids(e4m3):
    """Rows over 16 distinct keys sent to the exact repair (threshold above
    every score): the boundary tie resolves to the lowest tied ids there too
    (the checker applies the tie rule on the GPU's own scores)."""
    case = synth.causal_case("ties_repair", 8, 20000, seed=30, key_mode="ties16", K=300)
    log("case", case.name)
    r = run_prefill(case, scores=True, force_tau=float("inf"))
    st = r["stats"]
    log("stats", st)
    assert st["repaired"] == case.Q, st
    check_prefill_rows(case, r["out"], np.arange(case.Q), gpu_scores=r["scores"], e4m3=e4m3)


def test_tie_group_beyond_the_gather_through_repair(e4m3):
    """Rows over 16 distinct keys at 163840 keys sent to the exact repair:
    the K-th score is held by more keys than the repair gathers per row
    (8192), so its last step selects among them from the row's scratch
    keys; ties still resolve to the lowest ids."""
    pos = np.arange(163840 - 8, 163840, dtype=np.int64)
    case = synth.causal_case("ties_scratch", 8, 163840, seed=32, key_mode="ties16", positions=pos)
    log("case", case.name)
    r = run_prefill(case, scores=True, force_tau=float("inf"))
    st = r["stats"]
    log("stats", st)
    assert st["repaired"] == case.Q, st
    for t in range(case.Q):   # the case reaches that step: a tie group above the gather's capacity
        row = r["scores"][t, case.row_start[t]:case.row_end[t]]
        kth = np.partition(row, -case.K)[-case.K]
        assert np.count_nonzero(row == kth) > 8192, t
    check_prefill_rows(case, r["out"], np.arange(case.Q), gpu_scores=r["scores"], e4m3=e4m3)


def test_output_is_deterministic():
    """Two calls on the same inputs select the same ids (ties included)."""
    case = synth.causal_case("determinism", 16, 12000, seed=31, key_mode="ties16", K=512)
    log("case", case.name)
    a = run_prefill(case)["out"]
    b = run_prefill(case, force_tau=float("inf"))["out"]   # all rows through repair
    c = run_prefill(case)["out"]
    assert np.array_equal(np.sort(a, axis=1), np.sort(c, axis=1))
    assert np.array_equal(np.sort(a, axis=1), np.sort(b, axis=1))


def test_invalid_ranges_give_minus_one():
    case = synth.random_case("badrange", 6, 1000, seed=26, K=64, min_len=10)
    case.row_start[1], case.row_end[1] = 50, 40        # start > end
    case.row_end[4] = case.N + 5                        # end > N
    log("case", case.name)
    r = run_prefill(case)
    assert np.all(r["out"][1] == -1) and np.all(r["out"][4] == -1)
    assert r["stats"]["bad_rows"] == 2
    check_prefill_rows(case, r["out"], [0, 2, 3, 5])


def test_identical_keys_get_identical_scores():
    case = synth.causal_case("ties_small", 8, 6000, seed=27, key_mode="ties16", K=300)
    log("case", case.name)
    r = run_prefill(case, scores=True)
    keys = np.concatenate([case.k8, case.k_scale.view(np.uint8).reshape(-1, 4)], axis=1)
    _, group = np.unique(keys, axis=0, return_inverse=True)
    group = group.reshape(-1)
    for t in range(case.Q):
        s1 = case.row_end[t]
        S = r["scores"][t, :s1]
        for g in range(16):
            v = S[group[:s1] == g]
            assert v.size == 0 or np.all(v.view(np.uint32) == v[0].view(np.uint32))
    check_prefill_rows(case, r["out"], np.arange(case.Q))
