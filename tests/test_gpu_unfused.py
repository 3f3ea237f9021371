"""The unfused comparator on MI355X: the standalone dense-matrix top-K
(idx_topk_rows) against an exact CPU top-K of the same FP32 matrix, and the
unfused prefill (explicit score matrix, then top-K) against the fused path
and the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import check

pytestmark = pytest.mark.gpu

from gpu_util import check_prefill_rows, dev_prefill, log, sample_rows  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import scoring_exact_top_amd  # noqa: F401  (fails loudly if the library is missing)


def _rows(S, starts, ends, K):
    import scoring_exact_top_amd as lib
    d = torch.from_numpy(np.ascontiguousarray(S, dtype=np.float32)).cuda()
    out = lib.topk_rows(d, torch.from_numpy(starts.astype(np.int32)).cuda(),
                        torch.from_numpy(ends.astype(np.int32)).cuda(), K)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_rows(S, starts, ends, K, out, name):
    for t in range(S.shape[0]):
        s0, s1 = int(starts[t]), int(ends[t])
        if s0 < 0 or s0 > s1 or s1 > S.shape[1]:
            assert (out[t] == -1).all(), "%s row %d: invalid range not all -1" % (name, t)
            continue
        check.check_debug_canonical(out[t], S[t], s0, s1, K, where="%s row %d" % (name, t))


@pytest.mark.parametrize("K", [1, 100, 2048])
def test_rows_gaussian_ragged(K):
    """Gaussian rows with ragged, unaligned ranges: empty, shorter than K,
    exactly K, K+1, and long rows spanning several load steps with a tail."""
    rng = np.random.default_rng(40 + K)
    Q, N = 12, 21011
    S = rng.standard_normal((Q, N)).astype(np.float32)
    lens = [0, 1, K - 1, K, K + 1, 5000, 9999, 20000, N - 3, N, 7777, 12345]
    starts = np.array([min(N - L, int(rng.integers(0, N - L + 1))) for L in lens])
    ends = starts + np.array(lens)
    starts[-1], ends[-1] = 7, N                     # unaligned start, to the end
    log("rows", K, list(zip(starts.tolist(), ends.tolist())))
    out = _rows(S, starts, ends, K)
    _check_rows(S, starts, ends, K, out, "gauss K=%d" % K)


def test_rows_ties_and_bins():
    """Rows whose boundary bin holds more keys than fit on chip (the generic
    radix path): 16 distinct values, all values equal, +0/-0 mixtures; and a
    row whose values differ only in low mantissa bits (one top-11-bit bin)."""
    rng = np.random.default_rng(7)
    Q, N, K = 6, 30000, 2048
    vals = rng.standard_normal(16).astype(np.float32)
    S = np.empty((Q, N), dtype=np.float32)
    S[0] = vals[rng.integers(0, 16, N)]
    S[1] = 1.5
    S[2] = np.where(rng.random(N) < 0.5, np.float32(0.0), np.float32(-0.0))
    S[3] = (1.0 + rng.integers(0, 1 << 12, N) * 2.0 ** -23).astype(np.float32)
    S[4] = rng.standard_normal(N).astype(np.float32)
    S[4, ::3] = S[4, 100]                           # a third of the row tied at one value
    S[5] = -np.abs(rng.standard_normal(N)).astype(np.float32)
    starts = np.array([0, 3, 1, 0, 2, 5])
    ends = np.array([N, N - 1, N, 29999, N, N])
    out = _rows(S, starts, ends, K)
    _check_rows(S, starts, ends, K, out, "ties")


def _sample_mask(L):
    """Positions of the dense top-K's sample: 16 blocks of 256 scores, block j
    at j * ((L - 256) // 15) (restated here to build rows that fool it)."""
    step = (L - 256) // 15
    m = np.zeros(L, dtype=bool)
    for j in range(16):
        m[j * step: j * step + 256] = True
    return m


def test_rows_biased_samples_take_the_fallbacks():
    """Rows built against the sampled cut: 600 huge values inside the sample
    blocks (the cut keeps fewer than K keys: histogram over the whole row),
    and 9000 huge values outside them (the cut keeps more than fit: histogram
    above the cut), each with ragged, unaligned ranges."""
    rng = np.random.default_rng(11)
    N, K = 30000, 2048
    S = rng.standard_normal((4, N)).astype(np.float32)
    starts = np.array([0, 3, 0, 5])
    ends = np.array([N, N - 2, N, N - 1])
    for t in (0, 1):
        L = ends[t] - starts[t]
        inside = np.nonzero(_sample_mask(L))[0]
        S[t, starts[t] + rng.choice(inside, 600, replace=False)] = 50.0 + rng.random(600).astype(np.float32)
    for t in (2, 3):
        L = ends[t] - starts[t]
        outside = np.nonzero(~_sample_mask(L))[0]
        S[t, starts[t] + rng.choice(outside, 9000, replace=False)] = 50.0 + rng.random(9000).astype(np.float32)
    out = _rows(S, starts, ends, K)
    _check_rows(S, starts, ends, K, out, "biased")


def test_rows_invalid_ranges():
    S = np.zeros((3, 1000), dtype=np.float32)
    out = _rows(S, np.array([-1, 10, 5]), np.array([10, 5, 1001]), 16)
    assert (out == -1).all()


def _unfused(case, stats=False):
    import scoring_exact_top_amd as lib
    d = dev_prefill(case)
    ws = lib.alloc_workspace(lib.prefill_unfused_workspace_bytes(case.Q, case.N, case.K), "cuda")
    out = lib.prefill_unfused(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                              d["row_end"], case.K, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lib.read_stats(ws)


def _fused(case):
    import scoring_exact_top_amd as lib
    d = dev_prefill(case)
    out = lib.prefill(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                      d["row_end"], case.K)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _same_sets(a, b, name):
    sa, sb = np.sort(a, axis=1), np.sort(b, axis=1)
    bad = np.nonzero((sa != sb).any(axis=1))[0]
    assert bad.size == 0, "%s: unfused and fused selections differ on rows %s" % (name, bad[:10])


def test_unfused_ragged_matches_oracle_and_fused():
    case = synth.random_case("unfused_ragged", 37, 5000, seed=21, K=1000, min_len=0)
    case.row_end[3] = case.row_start[3]
    log("case", case.name)
    out, st = _unfused(case)
    check_prefill_rows(case, out, np.arange(case.Q))
    _same_sets(out, _fused(case), case.name)
    assert st["rows"] == case.Q and st["bad_rows"] == 0


@pytest.mark.parametrize("wl", ["prefill_smoke", "prefill_chunk", "long_prefill"])
def test_unfused_workloads_match_fused(wl):
    """Full workloads: every row's id set equals the fused path's (same
    scores, same tie rule); sampled rows against the oracle."""
    case = synth.WORKLOADS[wl](0)
    log("case", case.name)
    out, st = _unfused(case)
    _same_sets(out, _fused(case), case.name)
    rows = sample_rows(case.Q, 4 if case.Q > 64 else case.Q, seed=3)
    check_prefill_rows(case, out, rows)
    log(case.name, st)


def test_unfused_adversarial_ties_match_fused():
    """The adversarial tie rows (16 distinct key vectors) take the generic
    radix path of the dense top-K."""
    case = synth.adversarial(0)[0]
    log("case", case.name)
    out, st = _unfused(case)
    _same_sets(out, _fused(case), case.name)
    check_prefill_rows(case, out, sample_rows(case.Q, 3, seed=4))
    log(case.name, st)
    assert st["repaired"] > 0
