"""Full-configuration audits on MI355X: every row of the benchmarked prefill
workloads, in the benchmark's launch configuration, against the CPU oracle
(the correctness audit of the Fusing Indexer Scoring and Exact Top-k page,
"6.3 Correctness", extended from sampled rows to all of them).  Each
call also returns its per-row outcome, so the rows that the exact repair
rewrote are named and checked like every other.  Plus the paths that only
large inputs reach: failed rows beyond the repair slots, and a key count at
the addressing limit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import check

pytestmark = pytest.mark.gpu

from gpu_util import audit_rows, check_prefill_rows, log, run_prefill, status_matches_stats  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import scoring_exact_top_amd  # noqa: F401  (fails loudly if the library is missing)


def _audit(case):
    import scoring_exact_top_amd as lib
    log("case", case.name, case.Q, case.N)
    r = run_prefill(case, status=True)
    st, status = r["stats"], r["status"]
    log("stats", st)
    status_matches_stats(status, st)
    repaired = np.nonzero((status == lib.ROW_UNDERFLOW) | (status == lib.ROW_OVERFLOW))[0]
    log("rows repaired", repaired.tolist()[:40], "(%d)" % repaired.size)
    rep = audit_rows(case, r["out"])
    log(case.name, "every row matches the oracle", rep)
    assert rep["rows"] == case.Q
    return st, repaired


def test_audit_prefill_chunk_every_row():
    st, _ = _audit(synth.prefill_chunk(0))
    assert st["rows"] == 4096 and st["bad_rows"] == 0


def test_audit_long_prefill_every_row():
    st, repaired = _audit(synth.long_prefill(0))
    assert st["rows"] == 4096 and st["bad_rows"] == 0
    assert st["repaired"] == repaired.size


def test_audit_adversarial_every_row():
    """All four sub-calls: ties, the off-lattice outlier block (rows whose
    segments overflow with outliers scoring above the selection go through
    the exact repair), the on-lattice decoys (whose rows underflow and go
    through it too) and plain rows."""
    for case in synth.adversarial(0):
        st, repaired = _audit(case)
        if case.name == "adversarial_outlier":
            assert st["overflow"] > 0 and repaired.size == st["repaired"] > 0, st
        if case.name == "adversarial_decoy":
            assert st["underflow"] > 0 and repaired.size == st["repaired"] > 0, st
        if case.name == "adversarial_ties16":
            assert st["fast_ok"] >= 0.9 * case.Q, st


def test_repair_beyond_the_slots(e4m3_table):
    """More failed rows than the repair scratch has slots for: with N = 2^20
    keys the scratch holds 256 rows, so of 300 rows forced to fail (a
    threshold above every score) the last 44 are repaired whole by the
    fallback workgroups.  Every row against the oracle, and the selection
    bit-exact and canonical on the GPU's own scores."""
    import scoring_exact_top_amd as lib
    N, Q = 1 << 20, 300
    case = synth.random_case("repair_fallback", Q, N, seed=51, K=2048, min_len=2500, max_len=20000)
    log("case", case.name, Q, N)
    r = run_prefill(case, status=True, scores=True, force_tau=float("inf"))
    st = r["stats"]
    log("stats", st)
    status_matches_stats(r["status"], st)
    assert st["underflow"] == Q and st["repaired"] == Q, st
    rep = audit_rows(case, r["out"], batch=50, gpu_scores=r["scores"], e4m3=e4m3_table)
    log("fallback rows match the oracle", rep)
    del lib


def test_key_count_at_the_addressing_limit():
    """N at the largest accepted value ((N + 64) * 128 < 2^31): rows at the
    end of the key range put the main kernel's refills up to 32 tiles past
    the last tile, where their offsets would exceed 31 bits; those loads
    must read zeros, and the rows must match the oracle."""
    N = (2 ** 31 - 1) // 128 - 64
    ends = np.array([N, N, N - 1, N - 63, N - 64, N - 4000, N, N - 1], dtype=np.int64)
    lens = np.array([3000, 2100, 5000, 2048, 1, 2500, 9000, 64], dtype=np.int64)
    case = synth.random_codes_case("addr_limit", N, ends - lens, ends, seed=52, K=2048)
    log("case", case.name, case.Q, N)
    r = run_prefill(case, status=True)
    st = r["stats"]
    log("stats", st)
    status_matches_stats(r["status"], st)
    rep = check_prefill_rows(case, r["out"], np.arange(case.Q))
    log("rows at the limit match the oracle", rep)


def test_decode_debug_scores_on_the_paged_workload(e4m3_table):
    """Paged decode's debug entry returns the score rows its selection read:
    on the benchmarked batch they match the oracle element by element, and
    the selection is bit-exact (and follows the lowest-position tie rule) on
    those scores, mapped back from physical cache slots to logical
    positions."""
    import scoring_exact_top_amd as lib
    case = synth.paged_decode(0)
    log("case", case.name, case.seq_lens.tolist())
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = lib.alloc_workspace(lib.decode_workspace_bytes(case.B, case.max_pages, case.page_size, case.K), "cuda")
    S = torch.full((case.B, case.max_pages * 64), float("nan"), dtype=torch.float32, device="cuda")
    out = lib.decode_paged(t(case.q8), t(case.q_scale), t(case.k_cache), t(case.k_scale), t(case.w),
                           t(case.page_table), t(case.seq_lens), case.K, workspace=ws, scores_out=S)
    torch.cuda.synchronize()
    out, S = out.cpu().numpy(), S.cpu().numpy()
    topk, theta, sc = oracle.decode_case(case)
    scored = 0
    for b, L in enumerate(case.seq_lens):
        L = int(L)
        pt = case.page_table[b]
        phys = pt[np.arange(L) // 64].astype(np.int64) * 64 + np.arange(L) % 64
        inv = {int(p): i for i, p in enumerate(phys)}
        kk = min(case.K, L)
        logical = np.array([inv[int(x)] for x in out[b, :kk]] + [-1] * (case.K - kk), dtype=np.int64)
        where = "seq %d (L=%d)" % (b, L)
        check.check_selection(logical, sc[b], 0, L, case.K, theta[b], where=where)
        if L <= case.K:
            continue
        keys = case.k_cache.reshape(-1, 128)[phys]
        kscale = case.k_scale.reshape(-1)[phys]
        qs = np.ones(64) if case.q_scale is None else case.q_scale[b].astype(np.float64)
        B = check.bound_from_values(e4m3_table[case.q8[b]], e4m3_table[keys], case.w[b].astype(np.float64) * qs,
                                    kscale.astype(np.float64))
        cancel = check.check_scores(S[b, :L], sc[b, :L], bound=B, where=where)
        check.check_debug_bitexact(logical, S[b], 0, L, case.K, where=where)
        check.check_debug_canonical(logical, S[b], 0, L, case.K, where=where)
        log(where, "scores match the oracle (%d by the cancellation clause only)" % cancel)
        scored += 1
    assert scored == int(np.sum(case.seq_lens > case.K))
