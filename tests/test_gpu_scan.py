"""BF16 stream scan on MI355X against the CPU oracle: element-wise scores, the
selection tolerance, bit-exact selection on the GPU's own scores (lowest-id
tie rule), ragged stream lengths, ties, invalid lengths, and sampled streams
of the full 32 x 262144 workload."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import check

pytestmark = pytest.mark.gpu

from gpu_util import log  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import scoring_exact_top_amd  # noqa: F401  (fails loudly if the library is missing)


def _dec(a16):
    return torch.from_numpy(np.ascontiguousarray(a16).view(np.int16)).view(torch.bfloat16).double().numpy()


def _bound(case, b):
    """B[i] of stream b (the pinned check.bound_from_values, unit scales)."""
    return check.bound_from_values(_dec(case.q16[b]), _dec(case.k16[b, :case.lens[b]]), case.w[b].astype(np.float64))


def _run(case, scores=False):
    import scoring_exact_top_amd as lib
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = lib.alloc_workspace(lib.scan_bf16_workspace_bytes(case.B, case.N, case.K), "cuda")
    out = lib.scan_bf16(t(case.q16.view(np.int16)), t(case.w), t(case.k16.view(np.int16)), t(case.lens),
                        case.K, workspace=ws)
    torch.cuda.synchronize()
    S = lib.scan_bf16_scores(ws, case.B, case.N).cpu().numpy() if scores else None
    return out.cpu().numpy(), S, lib.read_stats(ws)


def _check(case, out, S, streams):
    valid = [b for b in streams if 0 <= case.lens[b] <= case.N]
    for b in streams:
        if b not in valid:
            assert (out[b] == -1).all(), "%s stream %d: invalid length must give -1" % (case.name, b)
    if not valid:
        return
    topk, theta, sc = oracle.scan_bf16(case.q16[valid], case.w[valid], case.k16[valid], case.lens[valid], case.K)
    for j, b in enumerate(valid):
        L = int(case.lens[b])
        where = "%s stream %d" % (case.name, b)
        check.check_selection(out[b], sc[j], 0, L, case.K, theta[j], where=where)
        if S is not None and L > case.K:
            check.check_scores(S[b, :L], sc[j, :L], bound=_bound(case, b), where=where)
            check.check_debug_bitexact(out[b], S[b], 0, L, case.K, where=where)
            check.check_debug_canonical(out[b], S[b], 0, L, case.K, where=where)


@pytest.mark.parametrize("K", [1, 100, 2048])
def test_scan_ragged_streams(K):
    lens = [0, 1, K, K + 1, 5000, 9001, 9001, 2049]
    case = synth.scan_case("scan_ragged", len(lens), 9001, seed=10 + K, lens=lens, K=K)
    log("case", case.name, lens, "K", K)
    out, S, st = _run(case, scores=True)
    log("stats", st)
    _check(case, out, S, list(range(case.B)))
    assert st["rows"] == case.B


def test_scan_ties_and_invalid_lengths():
    """Identical keys (the lowest positions win), and lengths outside [0, N]."""
    case = synth.scan_case("scan_ties", 4, 6000, seed=7, lens=[6000, 6000, -1, 6001], K=2048)
    case.k16[1] = case.k16[1, 123]                       # every key of stream 1 equal
    out, S, st = _run(case, scores=True)
    _check(case, out, S, [0, 1, 2, 3])
    assert sorted(out[1].tolist()) == list(range(2048))
    assert st["bad_rows"] == 2


def test_scan_full_workload_every_stream():
    """The 32 x 262144 workload in the benchmark's launch configuration: every
    stream against the oracle (selection tolerance, element-wise scores,
    bit-exact and canonical selection on the GPU's own scores)."""
    case = synth.bf16_scan(0)
    log("case", case.name)
    out, S, st = _run(case, scores=True)
    log("stats", st)
    for b0 in range(0, case.B, 8):
        _check(case, out, S, list(range(b0, min(case.B, b0 + 8))))
        log("streams", b0, "..", min(case.B, b0 + 8) - 1, "match the oracle")
    assert st["fast_ok"] == case.B


def test_stream_floor_values():
    """The floor kernel reads every record and writes the sum of words 0 and 3
    of its 16 quads (small integers, so the sum is exact in any order)."""
    import scoring_exact_top_amd as lib
    n = 3 * 1024 + 5
    rng = np.random.default_rng(3)
    src = rng.integers(-50, 50, size=(n, 64)).astype(np.float32)
    want = src.reshape(n, 16, 4)[:, :, [0, 3]].sum(axis=(1, 2))
    got = lib.stream_floor(torch.from_numpy(src).cuda()).cpu().numpy()
    assert np.array_equal(got, want)


def _sample_positions(L, blocks=16, width=256):
    """Positions the selection's sampled cut reads in a row of L scores
    (16 blocks of 256 consecutive keys, evenly spaced): used only to build
    inputs that push the cut off, the check stays the oracle's."""
    step = (L - width) // (blocks - 1)
    return np.concatenate([np.arange(j * step, j * step + width) for j in range(blocks)])


def _boost(k16_row, idx, factor):
    """Multiply the BF16 keys at idx by a power of two (exact in BF16)."""
    x = torch.from_numpy(k16_row[idx].view(np.int16)).view(torch.bfloat16) * factor
    k16_row[idx] = x.view(torch.int16).numpy().view(np.uint16)


def test_scan_biased_samples_take_the_fallbacks():
    """Nonnegative head weights make a key's score scale with the key.
    Stream 0: only the sampled keys boosted, so the cut lands above nearly
    every key and the gathered keys number fewer than K (underflow).  Stream
    1: every key but the sampled ones boosted, so the cut lands below almost
    the whole row and the gather overflows its capacity.  Both go through
    the in-kernel fallbacks and must still equal the oracle."""
    L = 30000
    case = synth.scan_case("scan_biased", 3, L, seed=21, K=2048)
    case.w[:] = np.abs(case.w)
    samp = _sample_positions(L)
    _boost(case.k16[0], samp, 8.0)
    rest = np.setdiff1d(np.arange(L), samp)
    _boost(case.k16[1], rest, 8.0)
    # the inputs do push the cut (r-th largest sample, r for about 2K keys
    # above it) as intended, on the oracle's scores
    _, _, sc = oracle.scan_bf16(case.q16[:2], case.w[:2], case.k16[:2], case.lens[:2], case.K)
    r = -(-2 * case.K * samp.size // L)
    above = [int((sc[b, :L] >= np.sort(sc[b, samp])[::-1][r - 1]).sum()) for b in range(2)]
    log("keys at or above the sampled cut", above)
    assert above[0] < case.K and above[1] > 6144
    out, S, st = _run(case, scores=True)
    log("stats", st)
    _check(case, out, S, [0, 1, 2])


def test_scan_longest_stream():
    """One stream of the most keys the ABI accepts ((N + 64) * 256 < 2^31):
    with a single stream, 1024 workgroups sweep it and each refill runs up
    to 4096 tiles past the current one, so the sweep's last refills fall far
    past the stream's end.  Full length and a ragged one, against the
    oracle."""
    import scoring_exact_top_amd as lib
    N = 0x7FFFFFFF // 256 - 64
    case = synth.scan_case("scan_longest", 1, N, seed=31, K=2048)
    log("case", case.name, N)
    dq, dw, dk = (torch.from_numpy(np.ascontiguousarray(a)).cuda()
                  for a in (case.q16.view(np.int16), case.w, case.k16.view(np.int16)))
    ws = lib.alloc_workspace(lib.scan_bf16_workspace_bytes(1, N, case.K), "cuda")
    for L in (N, N - 12345):
        lens = np.array([L], dtype=np.int32)
        out = lib.scan_bf16(dq, dw, dk, torch.from_numpy(lens).cuda(), case.K, workspace=ws)
        torch.cuda.synchronize()
        topk, theta, sc = oracle.scan_bf16(case.q16, case.w, case.k16, lens, case.K)
        check.check_selection(out.cpu().numpy()[0], sc[0], 0, L, case.K, theta[0],
                              where="longest stream, L=%d" % L)
