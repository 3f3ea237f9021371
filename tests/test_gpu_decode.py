"""Paged decode parity on MI355X against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import check
from gpu_util import log

pytestmark = pytest.mark.gpu


def _run(case, **opts):
    import scoring_exact_top_amd as lib
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = lib.alloc_workspace(lib.decode_workspace_bytes(case.B, case.max_pages, case.page_size, case.K),
                             "cuda")
    out = lib.decode_paged(t(case.q8), t(case.q_scale), t(case.k_cache), t(case.k_scale), t(case.w),
                           t(case.page_table), t(case.seq_lens), case.K, workspace=ws, **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lib.read_stats(ws)


def _check(case, out):
    topk, theta, sc = oracle.decode_case(case)
    for b, L in enumerate(case.seq_lens):
        L = int(L)
        pt = case.page_table[b]
        # map physical slots back to logical positions
        phys_of = lambda i: pt[i // 64] * 64 + i % 64
        inv = {int(phys_of(i)): i for i in range(L)}
        kk = min(case.K, L)
        o = out[b]
        assert np.all(o[kk:] == -1), b
        assert all(int(x) in inv for x in o[:kk]), b
        logical = np.array([inv[int(x)] for x in o[:kk]] + [-1] * (case.K - kk), dtype=np.int64)
        check.check_selection(logical, sc[b], 0, L, case.K, theta[b], where="seq %d" % b)


def test_paged_decode_workload():
    case = synth.paged_decode(0)
    log("case", case.name, case.seq_lens.tolist())
    out, st = _run(case)
    log("stats", st)
    assert st["rows"] == case.B and st["trivial"] == int(np.sum(case.seq_lens <= case.K))
    _check(case, out)


def test_decode_edges_and_q_scale():
    lens = [0, 1, 2047, 2048, 2049, 4095, 8192, 8193, 16384, 16385, 20000]
    case = synth.decode_case("edges", lens, seed=31, max_pages=400, with_q_scale=True)
    log("case", case.name, lens)
    out, st = _run(case)
    log("stats", st)
    _check(case, out)
    assert np.all(out[0] == -1)


def test_decode_bad_page_id():
    case = synth.decode_case("badpage", [3000, 5000], seed=32, max_pages=100)
    case.page_table[1, 3] = case.k_cache.shape[0] + 7
    out, st = _run(case)
    assert np.all(out[1] == -1) and st["bad_rows"] == 1


def test_decode_row_paths():
    """Sequence lengths around each limit of the per-sequence selection:
    around K, rows gathered whole (below 4096 keys), sampled rows (one-pass
    gather); every row exact, the counters add up."""
    lens = [1500, 2049, 3000, 4095, 4096, 9000, 16384, 20000, 65536]
    case = synth.decode_case("dec_paths", lens, seed=33, max_pages=1024)
    log("case", case.name, lens)
    out, st = _run(case)
    log("stats", st)
    scored = int(np.sum(case.seq_lens > case.K))
    assert st["fast_ok"] + st["repaired"] == scored and st["trivial"] == len(lens) - scored
    _check(case, out)


def test_decode_rejects_a_threshold():
    """Decode samples its threshold itself: the debug knob that forces one
    is refused, not ignored."""
    import scoring_exact_top_amd as lib
    case = synth.decode_case("dec_tau", [3000], seed=34, max_pages=100)
    with pytest.raises(lib.IdxTopkError):
        _run(case, force_tau=1.0)


def _tie_keys(case, seed):
    """Every key of the cache becomes one of 16 (code vector, scale) pairs."""
    rng = np.random.default_rng(seed)
    P, page, D = case.k_cache.shape
    pick = rng.integers(0, 16, P * page)
    codes = case.k_cache.reshape(-1, D)[rng.choice(P * page, 16, replace=False)].copy()
    scales = case.k_scale.reshape(-1)[rng.choice(P * page, 16, replace=False)].copy()
    case.k_cache = np.ascontiguousarray(codes[pick].reshape(P, page, D))
    case.k_scale = np.ascontiguousarray(scales[pick].reshape(P, page))
    return case


def test_decode_ties_take_the_lowest_positions():
    """Massive ties at the K-th score (16 distinct keys): the selected
    physical slots are those of the lowest tied logical positions; the tie
    group exceeds the on-chip gather, so the generic radix path runs."""
    lens = [3000, 20000, 60000]
    case = _tie_keys(synth.decode_case("dec_ties", lens, seed=36, max_pages=1000), 37)
    log("case", case.name, lens)
    out, st = _run(case)
    log("stats", st)
    _, theta, sc = oracle.decode_case(case)
    for b, L in enumerate(case.seq_lens):
        L = int(L)
        pt = case.page_table[b]
        inv = {int(pt[i // 64] * 64 + i % 64): i for i in range(L)}
        logical = np.array([inv[int(x)] for x in out[b][:min(case.K, L)]], dtype=np.int32)
        logical = np.concatenate([logical, np.full(case.K - logical.size, -1, np.int32)])
        check.check_debug_canonical(logical, sc[b].astype(np.float32), 0, L, case.K, where="seq %d" % b)


def test_decode_main_events_time_the_scoring_kernel():
    import scoring_exact_top_amd as lib
    case = synth.decode_case("dec_ev", [3000, 70000 // 2], seed=35, max_pages=600)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:  # torch creates the HIP event on first record
        e.record()
    out, st = _run(case, main_events=ev)
    assert ev[0].elapsed_time(ev[1]) > 0.0
    _check(case, out)


def test_decode_cache_beyond_2gib():
    """A page pool of more than 2 GiB of key codes (300000 pages of 64 keys):
    the sequences' pages sit above the 2 GiB mark, so every key read crosses
    it.  The same keys in a small pool give the oracle's reference."""
    import scoring_exact_top_amd as lib
    small = synth.decode_case("beyond_2gib", [5000, 3000, 70], seed=41, max_pages=100)
    P, base = 300000, 270000                    # 300000 * 64 * 128 B = 2.46 GB of codes
    assert (base * 64 * 128) > (1 << 31)
    log("case", small.name, "pool pages", P, "first used page", base)
    k_cache = torch.zeros((P, 64, 128), dtype=torch.uint8, device="cuda")
    k_scale = torch.ones((P, 64), dtype=torch.float32, device="cuda")
    n_small = small.k_cache.shape[0]                 # pages of the small pool
    k_cache[base: base + n_small] = torch.from_numpy(small.k_cache).cuda()
    k_scale[base: base + n_small] = torch.from_numpy(small.k_scale).cuda()
    table = np.where(small.page_table >= 0, small.page_table + base, -1).astype(np.int32)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = lib.alloc_workspace(lib.decode_workspace_bytes(small.B, small.max_pages, 64, small.K), "cuda")
    out = lib.decode_paged(t(small.q8), t(small.q_scale), k_cache, k_scale, t(small.w), t(table),
                           t(small.seq_lens), small.K, workspace=ws)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    shift = base * 64
    out = np.where(out >= 0, out - shift, -1)    # physical slots of the small pool
    _check(small, out)
    assert lib.read_stats(ws)["bad_rows"] == 0


def test_decode_large_batch_fixed_assignment():
    """300 sequences (beyond the 256 the balanced assignment plans for: a
    fixed number of scoring workgroups per sequence), ragged lengths around
    K, two of them with a bad page id."""
    g = np.random.default_rng(47)
    lens = g.integers(1, 5000, size=300).astype(np.int32)
    lens[:4] = [2048, 2049, 1, 4999]
    case = synth.decode_case("large_batch", lens, seed=47, max_pages=80)
    case.page_table[10, 0] = -5
    case.page_table[11, (int(case.seq_lens[11]) - 1) // 64] = 10 ** 7
    log("case", case.name, "B", case.B)
    out, st = _run(case)
    log("stats", st)
    assert (out[10] == -1).all() and (out[11] == -1).all()
    good = case.page_table.copy()
    keep = np.ones(case.B, dtype=bool)
    keep[[10, 11]] = False
    sub = synth.DecodeCase(case.name, case.q8[keep], None if case.q_scale is None else case.q_scale[keep],
                           case.k_cache, case.k_scale, case.w[keep], good[keep], case.seq_lens[keep],
                           case.page_size, case.K)
    _check(sub, out[keep])
    assert st["bad_rows"] == 2


def _sampled_pages(L):
    """Logical pages whose keys give a scored sequence of L keys its
    threshold (the sampling geometry documented with the decode scoring
    kernel: about one key in 200, as whole pages at a fixed stride over the
    full pages, at most 8; none up to 4096 keys).  Test construction only."""
    if L <= 4096:
        return []
    ns = -(-(L - 100) // 200)
    P = min(8, max(1, -(-ns // 64)))
    F = L // 64
    return [(2 * j + 1) * F // (2 * P) for j in range(P)]


def test_decode_boosted_sample_pages_force_underflow():
    """The keys of every sampled page scaled by 8: each sequence's threshold
    lands above nearly all its other keys, so fewer than K candidates pass
    it (underflow) and the selection falls back to the score row; exact."""
    lens = [9000, 30000, 65536]
    case = synth.decode_case("dec_decoy", lens, seed=38, max_pages=1024)
    for b, L in enumerate(lens):
        for lp in _sampled_pages(L):
            case.k_scale[case.page_table[b, lp]] *= 8.0
    log("case", case.name, lens, [len(_sampled_pages(L)) for L in lens], "sampled pages")
    out, st = _run(case)
    log("stats", st)
    assert st["underflow"] == len(lens) and st["fast_ok"] + st["repaired"] == len(lens)
    _check(case, out)


def test_decode_filtered_candidates_on_the_workload():
    """The benchmarked batch: every scored sequence is settled by the
    candidates its scoring kernel filtered (no fallback), and exact."""
    case = synth.paged_decode(0)
    out, st = _run(case)
    log("stats", st)
    scored = int(np.sum(case.seq_lens > case.K))
    assert st["fast_ok"] == scored and st["underflow"] == 0 and st["overflow"] == 0
    _check(case, out)


def test_decode_damped_sample_pages_force_overflow():
    """The keys of every sampled page scaled by 1/8: each sequence's
    threshold lands far below its K-th score, so about half its keys pass it,
    more than the selection holds in registers (counted as overflow), and
    the selection falls back to the score row; exact."""
    lens = [30000, 65536]
    case = synth.decode_case("dec_damped", lens, seed=39, max_pages=1024)
    for b, L in enumerate(lens):
        for lp in _sampled_pages(L):
            case.k_scale[case.page_table[b, lp]] *= 0.125
    out, st = _run(case)
    log("stats", st)
    assert st["overflow"] == len(lens) and st["fast_ok"] + st["repaired"] == len(lens)
    _check(case, out)


def test_decode_largest_filtered_batch():
    """256 sequences, the largest batch whose scoring kernel samples and
    filters (one fewer would change nothing, one more takes the pre-gather):
    ragged lengths around K, around the keep-every-key bound (4096) and up to
    20000, with the balanced plan giving some sequences one or two scoring
    workgroups; every sequence exact."""
    g = np.random.default_rng(49)
    lens = g.integers(1, 20000, size=256).astype(np.int32)
    lens[:8] = [2048, 2049, 4095, 4096, 4097, 4160, 1, 0]
    case = synth.decode_case("dec_b256", lens, seed=49, max_pages=320)
    log("case", case.name, "B", case.B)
    out, st = _run(case)
    log("stats", st)
    scored = int(np.sum(case.seq_lens > case.K))
    assert st["rows"] == case.B and st["fast_ok"] + st["repaired"] == scored
    # segments sized for the batch (8 B pairs per wave): nearly every
    # sequence is settled by its filtered candidates
    assert st["overflow"] + st["underflow"] <= scored // 50
    _check(case, out)
