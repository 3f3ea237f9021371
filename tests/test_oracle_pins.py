"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test ties one part of the oracle to a library routine, a closed form,
exact integer arithmetic or brute force, chosen so that a plausible slip (a
dropped ReLU, a sign, a wrong scale, a transposed operand, an index off by
the range start, a broken tie rule) fails at least one of them.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import check
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3(codes):
    t = torch.as_tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.float().double().numpy()


def _finite_codes(rng, shape, nonneg=False):
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    c = np.where((c & 0x7F) == 0x7F, c ^ 0x01, c)  # avoid the two NaN codes
    if nonneg:
        c &= 0x7F
    return c.astype(np.uint8)


def _case(q8, qs, k8, ks, w, rs, re, K):
    return synth.PrefillCase("pin", np.ascontiguousarray(q8), np.ascontiguousarray(qs, np.float32),
                             np.ascontiguousarray(k8), np.ascontiguousarray(ks, np.float32),
                             np.ascontiguousarray(w, np.float32), np.asarray(rs, np.int32),
                             np.asarray(re, np.int32), K)


# --------------------------------------------------------------- e4m3 decode

def test_e4m3_exhaustive_vs_torch(e4m3_table):
    ref = _torch_e4m3(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(e4m3_table), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(e4m3_table[~nan], ref[~nan])
    # sign of zero
    assert np.signbit(e4m3_table[0x80]) and not np.signbit(e4m3_table[0x00])


def test_e4m3_spec_points(e4m3_table):
    with open(os.path.join(GOLDEN, "e4m3_spec_points.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, val = line.split()
            v = float(val)
            got = e4m3_table[int(code, 16)]
            if np.isnan(v):
                assert np.isnan(got)
            else:
                assert got == v and np.signbit(got) == np.signbit(v), (code, got, v)
    assert np.nanmax(np.abs(e4m3_table)) == 448.0


# ------------------------------------------------------------ exact dot product

def test_dot_raw_exact_vs_integer_arithmetic():
    rng = np.random.default_rng(1)
    for _ in range(200):
        a = _finite_codes(rng, 128)
        b = _finite_codes(rng, 128)
        # every e4m3 value is n * 2^-9 with integer n: exact rational sum
        na = [int(Fraction(float(v)) * 512) for v in _torch_e4m3(a)]
        nb = [int(Fraction(float(v)) * 512) for v in _torch_e4m3(b)]
        exact = Fraction(sum(x * y for x, y in zip(na, nb)), 1 << 18)
        assert Fraction(oracle.dot_raw(a, b)) == exact


def test_dot_raw_extremes():
    a = np.full(128, 0x7E, np.uint8)       # 448
    b = np.full(128, 0xFE, np.uint8)       # -448
    assert oracle.dot_raw(a, b) == -128 * 448.0 * 448.0
    s = np.full(128, 0x01, np.uint8)       # 2^-9
    assert oracle.dot_raw(s, s) == 128 * 2.0 ** -18


# ------------------------------------------------------------ scoring closed forms

def test_one_hot_head_and_dim_gives_relu_of_key_column():
    """w = e_j, q[t,j] = e_d, scales 1  =>  I[s] = ReLU(dec(k8[s,d]))."""
    rng = np.random.default_rng(2)
    N, K = 300, 50
    for j, d in [(0, 0), (17, 77), (63, 127)]:
        q8 = _finite_codes(rng, (1, 64, 128))
        q8[0, j, :] = 0
        q8[0, j, d] = 0x38
        w = np.zeros((1, 64), np.float32)
        w[0, j] = 1.0
        k8 = _finite_codes(rng, (N, 128))
        case = _case(q8, np.ones((1, 64)), k8, np.ones(N), w, [0], [N], K)
        topk, theta, sc = oracle.prefill_case(case)
        col = np.maximum(_torch_e4m3(k8[:, d]), 0.0)
        assert np.array_equal(sc[0], col)
        assert np.array_equal(np.sort(col[topk[0]]), np.sort(col)[-K:])


def test_relu_even_odd_heads_gives_abs():
    """Heads alternate q = +e_0 / -e_0, w = 1: I = 32 max(c,0) + 32 max(-c,0) = 32|c|."""
    rng = np.random.default_rng(3)
    N = 256
    q8 = np.zeros((1, 64, 128), np.uint8)
    q8[0, 0::2, 0] = 0x38
    q8[0, 1::2, 0] = 0xB8
    k8 = np.zeros((N, 128), np.uint8)
    k8[:, 0] = _finite_codes(rng, N)
    ks = rng.uniform(0.5, 2.0, N).astype(np.float32)
    case = _case(q8, np.ones((1, 64)), k8, ks, np.ones((1, 64)), [0], [N], 16)
    _, _, sc = oracle.prefill_case(case)
    expect = 32.0 * np.abs(_torch_e4m3(k8[:, 0])) * ks.astype(np.float64)
    assert np.allclose(sc[0], expect, rtol=1e-15, atol=0)


def test_linear_regime_matches_matvec():
    """Nonnegative codes and w >= 0 keep every ReLU active, so
    I[s] = k_scale[s] * (sum_j w_j q_scale_j dec(q_j)) . dec(k_s)."""
    rng = np.random.default_rng(4)
    Q, N = 3, 500
    q8 = _finite_codes(rng, (Q, 64, 128), nonneg=True)
    k8 = _finite_codes(rng, (N, 128), nonneg=True)
    qs = rng.uniform(0.01, 1.0, (Q, 64)).astype(np.float32)
    ks = rng.uniform(0.01, 1.0, N).astype(np.float32)
    w = np.abs(rng.normal(0, 0.125, (Q, 64))).astype(np.float32)
    case = _case(q8, qs, k8, ks, w, [0] * Q, [N] * Q, 64)
    _, _, sc = oracle.prefill_case(case)
    qd = _torch_e4m3(q8)
    kd = _torch_e4m3(k8)
    for t in range(Q):
        u = (w[t].astype(np.float64) * qs[t]) @ qd[t]        # [128]
        expect = ks.astype(np.float64) * (kd @ u)
        assert np.allclose(sc[t], expect, rtol=1e-12, atol=0)


@pytest.mark.parametrize("sign", [1, -1, 0])
def test_scale_only_variation_orders_by_scale(sign):
    """All keys share one code vector and differ only in k_scale = c_s, so
    I[s] = c_s * I_u: top-K = K largest c_s (I_u > 0), K smallest (I_u < 0),
    all tied (I_u = 0)."""
    rng = np.random.default_rng(5)
    N, K = 1000, 100
    q8 = _finite_codes(rng, (1, 64, 128))
    u = _finite_codes(rng, 128)
    k8 = np.tile(u, (N, 1))
    c = rng.permutation(np.linspace(0.1, 10.0, N)).astype(np.float32)
    w = rng.normal(0, 0.125, (1, 64)).astype(np.float32)
    case = _case(q8, np.ones((1, 64)), k8, np.ones(N), w, [0], [N], K)
    _, _, s1 = oracle.prefill_case(case)
    I_u = s1[0, 0]
    if I_u == 0:
        pytest.skip("degenerate draw")
    w = w * (np.sign(I_u) * sign)
    case = _case(q8, np.ones((1, 64)), k8, c, w, [0], [N], K)
    topk, _, sc = oracle.prefill_case(case)
    if sign > 0:
        expect = np.argsort(-c)[:K]
    elif sign < 0:
        expect = np.argsort(c)[:K]
    else:
        assert np.all(sc[0] == 0) and not np.any(np.signbit(sc[0]))
        expect = np.arange(K)  # oracle's deterministic tie rule: lowest ids
    assert set(topk[0].tolist()) == set(expect.tolist())


# ------------------------------------------------------------------ selection

def test_selection_brute_force_tiny():
    """For N <= 10, K <= 5: the oracle's set is one of the K-subsets S with
    min(I[S]) >= max(I[rest]); with the lowest-id rule it is the
    lexicographically smallest such set."""
    rng = np.random.default_rng(6)
    for trial in range(60):
        N = int(rng.integers(1, 11))
        K = int(rng.integers(1, 6))
        q8 = _finite_codes(rng, (1, 64, 128))
        # a few distinct key vectors so that ties happen
        base = _finite_codes(rng, (3, 128))
        k8 = base[rng.integers(0, 3, N)]
        s0 = int(rng.integers(0, N))
        s1 = int(rng.integers(s0, N + 1))
        case = _case(q8, np.ones((1, 64)), k8, np.ones(N), rng.normal(0, .125, (1, 64)),
                     [s0], [s1], K)
        topk, theta, sc = oracle.prefill_case(case)
        L = s1 - s0
        kk = min(K, L)
        ids = list(range(s0, s1))
        valid_sets = []
        for S in itertools.combinations(ids, kk):
            rest = [i for i in ids if i not in S]
            if kk == 0 or not rest or min(sc[0][list(S)]) >= max(sc[0][rest]):
                valid_sets.append(S)
        got = tuple(sorted(topk[0][:kk].tolist()))
        assert got in valid_sets
        assert got == min(valid_sets)
        assert np.all(topk[0][kk:] == -1)
        if kk:
            assert theta[0] == np.sort(sc[0][s0:s1])[::-1][kk - 1]


def test_topk_values_match_torch_topk():
    case = synth.random_case("pin_topk", 6, 3000, seed=7, K=300, min_len=0)
    topk, theta, sc = oracle.prefill_case(case)
    for r in range(case.Q):
        s0, s1 = case.row_start[r], case.row_end[r]
        kk = min(case.K, s1 - s0)
        got = np.sort(sc[r][topk[r][:kk]])
        ref = torch.topk(torch.from_numpy(sc[r][s0:s1].copy()), kk).values.numpy()
        assert np.array_equal(got, np.sort(ref))
        check.check_exact_values(topk[r], sc[r], s0, s1, case.K)


def test_ties16_closed_form():
    """Keys from 16 distinct vectors: scores take <= 16 values; theta and the
    number taken at theta follow from the multiplicities crossing K."""
    case = synth.causal_case("pin_ties", 4, 6000, seed=8, key_mode="ties16", K=700)
    topk, theta, sc = oracle.prefill_case(case)
    keys = np.concatenate([case.k8, case.k_scale.view(np.uint8).reshape(-1, 4)], axis=1)
    uniq, group = np.unique(keys, axis=0, return_inverse=True)
    group = group.reshape(-1)
    assert len(uniq) == 16
    for r in range(case.Q):
        s0, s1 = case.row_start[r], case.row_end[r]
        vals = {}
        for g in range(16):
            ids = np.nonzero(group[s0:s1] == g)[0] + s0
            if ids.size:
                v = sc[r][ids]
                assert np.all(v == v[0])  # identical keys, identical scores
                vals.setdefault(float(v[0]), 0)
                vals[float(v[0])] += ids.size
        cum = 0
        for v in sorted(vals, reverse=True):
            if cum + vals[v] >= case.K:
                th, at = v, case.K - cum
                break
            cum += vals[v]
        assert theta[r] == th
        sel = sc[r][topk[r]]
        assert int(np.sum(sel == th)) == at
        assert int(np.sum(sel > th)) == case.K - at


# ------------------------------------------------------------------ checker

def test_checker_rejects_mutations():
    case = synth.random_case("pin_check", 3, 4000, seed=9, K=256, min_len=1000)
    topk, theta, sc = oracle.prefill_case(case)
    r = 0
    s0, s1, K = int(case.row_start[r]), int(case.row_end[r]), case.K
    good = topk[r].copy()
    check.check_selection(good, sc[r], s0, s1, K, theta[r])
    check.check_exact_values(good, sc[r], s0, s1, K)

    def bad(m):
        with pytest.raises(check.CheckError):
            check.check_selection(m, sc[r], s0, s1, K, theta[r])

    m = good.copy(); m[5] = m[6]; bad(m)                       # duplicate
    m = good.copy(); m[3] = s1; bad(m)                          # out of range (end)
    m = good.copy(); m[3] = s0 - 1; bad(m)                      # out of range (start)
    m = good.copy(); m[7] = -1; bad(m)                          # wrong count
    rest = np.setdiff1d(np.arange(s0, s1), good)
    low = rest[np.argmin(sc[r][rest])]
    m = good.copy(); m[0] = low; bad(m)                         # swapped-in lower element
    with pytest.raises(check.CheckError):
        check.check_exact_values(m, sc[r], s0, s1, K)
    # short row: wrong padding
    short = synth.random_case("pin_check2", 1, 300, seed=10, K=256, min_len=10, max_len=100)
    t2, th2, sc2 = oracle.prefill_case(short)
    a, b = int(short.row_start[0]), int(short.row_end[0])
    check.check_selection(t2[0], sc2[0], a, b, 256, th2[0])
    m = t2[0].copy(); m[-1] = a
    with pytest.raises(check.CheckError):
        check.check_selection(m, sc2[0], a, b, 256, th2[0])


def test_checker_score_tolerance_and_bitexact():
    case = synth.random_case("pin_tol", 2, 2000, seed=11, K=128, min_len=500)
    topk, theta, sc = oracle.prefill_case(case)
    s0, s1 = int(case.row_start[0]), int(case.row_end[0])
    I = sc[0][s0:s1]
    check.check_scores(I * (1 + 5e-4), I)
    with pytest.raises(check.CheckError):
        check.check_scores(I * (1 + 5e-3) + 1e-3, I)
    S = np.full(case.N, np.nan, np.float32)
    S[s0:s1] = I.astype(np.float32)
    sel, _ = oracle.topk_of_scores(S[s0:s1].astype(np.float64), 128)
    out = (sel + s0).astype(np.int32)
    check.check_debug_bitexact(out, S, s0, s1, 128)
    rest = np.setdiff1d(np.arange(s0, s1), out)
    m = out.copy(); m[0] = rest[0]
    with pytest.raises(check.CheckError):
        check.check_debug_bitexact(m, S, s0, s1, 128)


def test_checker_canonical_tie_rule():
    """A 60-way tie straddling the K-th place (24 ids above it, K = 64): only
    the 40 lowest tied ids are accepted.  Swapping in a higher tied id still
    gives a valid top-K (the bit-exact check passes) but breaks the rule."""
    rng = np.random.default_rng(5)
    s0, s1, K = 10, 410, 64
    ids = rng.permutation(np.arange(s0, s1))
    above, tied, rest = ids[:24], np.sort(ids[24:84]), ids[84:]
    S = np.full(500, np.nan, np.float32)
    S[above] = 2.0 + np.arange(24, dtype=np.float32) / 64
    S[tied] = 1.5
    S[rest] = rng.uniform(0.0, 1.0, rest.size).astype(np.float32)
    good = np.concatenate([above, tied[:40]]).astype(np.int32)
    check.check_debug_canonical(good, S, s0, s1, K)
    bad = good.copy()
    bad[-1] = tied[-1]
    check.check_debug_bitexact(bad, S, s0, s1, K)
    with pytest.raises(check.CheckError):
        check.check_debug_canonical(bad, S, s0, s1, K)


# ------------------------------------------------------------------ decode

def test_decode_trivial_path_is_a_remap():
    """seq_len <= K: every position is selected; ids are physical slots
    page_table[b][i // page] * page + i % page."""
    case = synth.decode_case("pin_dec_short", [1, 63, 64, 65, 700, 2048], seed=12,
                             max_pages=40)
    topk, theta, _ = oracle.decode_case(case)
    for b, L in enumerate(case.seq_lens):
        i = np.arange(L)
        phys = case.page_table[b][i // 64] * 64 + i % 64
        assert set(topk[b][:L].tolist()) == set(phys.tolist())
        assert np.all(topk[b][L:] == -1)


def test_decode_matches_prefill_on_gathered_keys():
    """The paged decode oracle equals the prefill oracle on the keys gathered
    into logical order, with ids mapped to physical slots."""
    case = synth.decode_case("pin_dec", [5000, 3000, 130], seed=13, K=500, with_q_scale=True)
    topk, theta, sc = oracle.decode_case(case)
    flat_k = case.k_cache.reshape(-1, 128)
    flat_s = case.k_scale.reshape(-1)
    for b, L in enumerate(case.seq_lens):
        i = np.arange(L)
        phys = case.page_table[b][i // 64] * 64 + i % 64
        pc = _case(case.q8[b:b + 1], case.q_scale[b:b + 1], flat_k[phys], flat_s[phys],
                   case.w[b:b + 1], [0], [L], case.K)
        t2, th2, s2 = oracle.prefill_case(pc)
        assert np.array_equal(s2[0], sc[b][:L])
        kk = min(L, case.K)
        assert np.array_equal(phys[t2[0][:kk]], topk[b][:kk])
        assert th2[0] == theta[b]


# ------------------------------------------------------------- BF16 stream scan

def _to_bf16_bits(x) -> np.ndarray:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16).copy()


def test_bf16_decode_exhaustive_vs_torch():
    """Every 16-bit pattern decodes to torch's bfloat16 -> float32 value (NaNs
    to NaN): BF16 is the upper half of an IEEE binary32."""
    bits = np.arange(65536, dtype=np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert oracle.bf16_value(0x3F80) == 1.0 and oracle.bf16_value(0xC040) == -3.0
    assert oracle.bf16_value(0x0001) == 2.0 ** -133          # smallest subnormal


def test_scan_one_hot_gives_relu_of_key_column():
    """Query head j0 = e_d0, all other heads zero, w = e_j0: every score is
    ReLU(k[i, d0]); the top-K follows that column (ties to lower positions)."""
    rng = np.random.default_rng(3)
    N, K, j0, d0 = 700, 50, 17, 93
    q = np.zeros((1, 64, 128), dtype=np.float32)
    q[0, j0, d0] = 1.0
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, j0] = 1.0
    kf = rng.standard_normal((1, N, 128)).astype(np.float32)
    k16 = _to_bf16_bits(kf)
    col = torch.from_numpy(k16[0, :, d0].view(np.int16)).view(torch.bfloat16).double().numpy()
    topk, theta, sc = oracle.scan_bf16(_to_bf16_bits(q), w, k16, np.array([N], np.int32), K)
    assert np.array_equal(sc[0], np.maximum(col, 0.0))
    order = sorted(range(N), key=lambda i: (-max(col[i], 0.0), i))
    assert topk[0].tolist() == order[:K]


def test_scan_linear_regime_matches_matvec():
    """Nonnegative queries, keys and weights: ReLU is the identity, so every
    score is one float64 matrix-vector product (sum_j w_j q_j) . k."""
    rng = np.random.default_rng(4)
    B, N = 2, 300
    q16 = _to_bf16_bits(np.abs(rng.standard_normal((B, 64, 128))))
    k16 = _to_bf16_bits(np.abs(rng.standard_normal((B, N, 128))))
    w = np.abs(rng.standard_normal((B, 64))).astype(np.float32)
    dec = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()
    _, _, sc = oracle.scan_bf16(q16, w, k16, np.array([N, N - 7], np.int32), 10)
    for b in range(B):
        u = (w[b].astype(np.float64)[:, None] * dec(q16[b])).sum(axis=0)
        want = dec(k16[b]) @ u
        L = N if b == 0 else N - 7
        np.testing.assert_allclose(sc[b, :L], want[:L], rtol=1e-12, atol=0)
        assert np.isnan(sc[b, L:]).all()


def test_scan_equals_fp8_oracle_on_common_values():
    """Values exactly representable in both e4m3 and BF16 (every e4m3 value
    is): with unit scales the FP8 prefill oracle and the BF16 scan oracle are
    two independent decodes of the same numbers, and must agree bit for bit
    on every score and on the selection."""
    rng = np.random.default_rng(5)
    N, K = 900, 64
    e4 = oracle.e4m3_table()
    codes_q = rng.integers(0, 256, (1, 64, 128)).astype(np.uint8)
    codes_k = rng.integers(0, 256, (N, 128)).astype(np.uint8)
    for c in (codes_q, codes_k):
        c[(c & 0x7F) == 0x7F] = 0x38                          # no NaN codes
    w = rng.standard_normal((1, 64)).astype(np.float32)
    pc = synth.PrefillCase("common", codes_q, np.ones((1, 64), np.float32), codes_k,
                           np.ones(N, np.float32), w, np.array([0], np.int32), np.array([N], np.int32), K)
    tk8, th8, sc8 = oracle.prefill_case(pc)
    q16 = _to_bf16_bits(e4[codes_q])
    k16 = _to_bf16_bits(e4[codes_k])[None]
    assert np.array_equal(torch.from_numpy(k16.view(np.int16)).view(torch.bfloat16).double().numpy()[0],
                          e4[codes_k])                        # the BF16 copies are exact
    tk16, th16, sc16 = oracle.scan_bf16(q16, w, k16, np.array([N], np.int32), K)
    assert np.array_equal(sc8[0], sc16[0]) and np.array_equal(tk8[0], tk16[0]) and th8[0] == th16[0]


def test_scan_ties_and_short_streams():
    """Identical keys tie: the K lowest positions; a stream with lens <= K
    returns all its positions then -1."""
    rng = np.random.default_rng(6)
    N, K = 500, 100
    q16 = _to_bf16_bits(rng.standard_normal((2, 64, 128)))
    w = rng.standard_normal((2, 64)).astype(np.float32)
    one = _to_bf16_bits(rng.standard_normal((1, 1, 128)))
    k16 = np.repeat(np.repeat(one, N, axis=1), 2, axis=0)
    topk, _, _ = oracle.scan_bf16(q16, w, k16, np.array([N, 60], np.int32), K)
    assert topk[0].tolist() == list(range(K))
    assert topk[1].tolist() == list(range(60)) + [-1] * (K - 60)


# ------------------------------------------------- cancellation-clause bound
#
# B[s] = k_scale[s] * sum_j |w_j q_scale_j| * sum_d |dec(q)_jd| |dec(k)_sd| is the
# magnitude behind the cancellation clause of check_scores.  The pins below tie
# check.bound_from_values (and the FP8 wrapper score_bound) to facts outside
# it; the mutants are plausible slips, and each must fail at least one pin.

def _bound_ok(q8, qs, k8, ks, w, t, ids, table, bound_fn):
    return bound_fn(table[q8[t]], table[k8[ids]], w[t].astype(np.float64) * qs[t].astype(np.float64),
                    ks[ids].astype(np.float64))


def _pin_linear_regime(bound_fn, table):
    """Nonnegative codes, w >= 0: no ReLU is active and no term cancels, so B
    equals the oracle's own score I (to fp64 rounding of the head sum)."""
    rng = np.random.default_rng(40)
    Q, N = 2, 300
    q8 = _finite_codes(rng, (Q, 64, 128), nonneg=True)
    k8 = _finite_codes(rng, (N, 128), nonneg=True)
    qs = rng.uniform(0.01, 1.0, (Q, 64)).astype(np.float32)
    ks = rng.uniform(0.01, 4.0, N).astype(np.float32)
    w = np.abs(rng.normal(0, 0.125, (Q, 64))).astype(np.float32)
    case = _case(q8, qs, k8, ks, w, [0] * Q, [N] * Q, 32)
    _, _, sc = oracle.prefill_case(case)
    ids = np.arange(N)
    return all(np.allclose(_bound_ok(q8, qs, k8, ks, w, t, ids, table, bound_fn), sc[t], rtol=1e-13, atol=0)
               for t in range(Q))


def _pin_head_pair(bound_fn, table):
    """Heads 0 and 1 hold q and -q (sign bit flipped), weights a > 0 and -b < 0,
    all other weights 0.  Closed form, summed term by term in exact rational
    arithmetic from torch's e4m3 decode:
        B[s] = ks[s] * (a qs0 + b qs1) * sum_d |q_d| |k_sd|
    which differs from |I[s]| = ks[s] |a qs0 relu(c) - b qs1 relu(-c)| whenever
    the products q_d k_sd have mixed signs."""
    rng = np.random.default_rng(41)
    N = 40
    q8 = np.zeros((1, 64, 128), np.uint8)
    qrow = _finite_codes(rng, 128)
    q8[0, 0] = qrow
    q8[0, 1] = qrow ^ 0x80
    k8 = _finite_codes(rng, (N, 128))
    qs = np.ones((1, 64), np.float32)
    qs[0, 0], qs[0, 1] = 0.75, 1.25
    ks = rng.uniform(0.5, 2.0, N).astype(np.float32)
    w = np.zeros((1, 64), np.float32)
    w[0, 0], w[0, 1] = 0.375, -0.625
    qd = _torch_e4m3(qrow)
    kd = _torch_e4m3(k8)
    hw = Fraction(float(w[0, 0])) * Fraction(float(qs[0, 0])) - Fraction(float(w[0, 1])) * Fraction(float(qs[0, 1]))
    want = np.array([float(Fraction(float(ks[s])) * hw *
                           sum(abs(Fraction(float(qd[d]))) * abs(Fraction(float(kd[s, d]))) for d in range(128)))
                     for s in range(N)])
    got = _bound_ok(q8, qs, k8, ks, w, 0, np.arange(N), table, bound_fn)
    return np.allclose(got, want, rtol=1e-14, atol=0)


def _pin_dominates(bound_fn, table):
    """|I| <= B on random signed data (triangle inequality), and B is not
    off by a factor of heads or dims: with unit-variance q and k and w of
    standard deviation sigma, B ~ 64 * 0.8 sigma * 128 * (2/pi) ~ 4200 sigma
    while a typical |I| ~ sqrt(64) * sigma * sqrt(E relu(c)^2) * 0.8 ~ 50 sigma,
    so the median ratio B/|I| sits near 100; it must stay in [30, 400]."""
    case = synth.random_case("pin_bound", 3, 1500, seed=42, K=64, min_len=1500)
    _, _, sc = oracle.prefill_case(case)
    ok = True
    for t in range(case.Q):
        ids = np.arange(case.N)
        B = _bound_ok(case.q8, case.q_scale, case.k8, case.k_scale, case.w, t, ids, table, bound_fn)
        I = sc[t]
        ok &= bool(np.all(np.abs(I) <= B * (1 + 1e-12)))
        ratio = np.median(B / np.maximum(np.abs(I), 1e-300))
        ok &= bool(30.0 < ratio < 400.0)
    return ok


_BOUND_PINS = [_pin_linear_regime, _pin_head_pair, _pin_dominates]


def _mut_no_kscale(qd, kd, wq, ks=None):
    return check.bound_from_values(qd, kd, wq, None)


def _mut_no_abs_codes(qd, kd, wq, ks=None):
    b = (np.asarray(kd, np.float64) @ np.asarray(qd, np.float64).T) @ np.abs(wq)
    return b * ks


def _mut_no_abs_weights(qd, kd, wq, ks=None):
    b = (np.abs(kd) @ np.abs(qd).T) @ np.asarray(wq, np.float64)
    return b * ks


def _mut_heads_summed_first(qd, kd, wq, ks=None):
    # sums the weighted query over heads before taking magnitudes (the wrong axis order)
    u = np.abs(np.asarray(wq, np.float64) @ np.asarray(qd, np.float64))
    return (np.abs(kd) @ u) * ks


def _mut_abs_after_dot(qd, kd, wq, ks=None):
    # |sum_d q k| instead of sum_d |q k|
    b = np.abs(np.asarray(kd, np.float64) @ np.asarray(qd, np.float64).T) @ np.abs(wq)
    return b * ks


def test_score_bound_pins(e4m3_table):
    for pin in _BOUND_PINS:
        assert pin(check.bound_from_values, e4m3_table), pin.__name__


def test_score_bound_wrapper_matches_its_definition(e4m3_table):
    """score_bound(row t, ids) is bound_from_values on row t's decoded codes,
    with w*q_scale and the keys' scales (and all-ones q_scale when None)."""
    case = synth.random_case("pin_bound_wrap", 2, 700, seed=43, K=64, min_len=700)
    ids = np.array([0, 5, 699, 350])
    for qs in (case.q_scale, None):
        B = check.score_bound(case.q8, qs, case.k8, case.k_scale, case.w, 1, ids, e4m3_table)
        qsr = np.ones(64) if qs is None else qs[1].astype(np.float64)
        want = [float(case.k_scale[s]) * sum(abs(float(case.w[1, j]) * qsr[j]) *
                                             sum(abs(e4m3_table[case.q8[1, j, d]] * e4m3_table[case.k8[s, d]])
                                                 for d in range(128)) for j in range(64)) for s in ids]
        assert np.allclose(B, want, rtol=1e-12, atol=0)


@pytest.mark.parametrize("mutant", [_mut_no_kscale, _mut_no_abs_codes, _mut_no_abs_weights,
                                    _mut_heads_summed_first, _mut_abs_after_dot])
def test_score_bound_mutants_fail_a_pin(mutant, e4m3_table):
    assert not all(pin(mutant, e4m3_table) for pin in _BOUND_PINS), mutant.__name__


def test_check_scores_cancellation_clause():
    """Where I cancels to zero the relative clause cannot hold, so the bound
    decides: an error of GAMMA*B/2 passes, 2*GAMMA*B fails; without a bound
    both fail.  Where |I| is large the relative clause decides alone."""
    g = check.GAMMA
    I = np.array([0.0, 0.0, 1e-9])
    B = np.array([10.0, 3.0, 7.0])
    assert check.check_scores(I + 0.5 * g * B, I, bound=B) == 3
    assert check.check_scores(I - 0.5 * g * B, I, bound=B) == 3
    with pytest.raises(check.CheckError):
        check.check_scores(I + 2.0 * g * B, I, bound=B)
    with pytest.raises(check.CheckError):
        check.check_scores(I + 0.5 * g * B, I)
    big = np.array([100.0])
    assert check.check_scores(big * (1 + 0.9 * check.REL_TOL), big, bound=np.array([1.0])) == 0
    with pytest.raises(check.CheckError):
        check.check_scores(big * (1 + 1.1 * check.REL_TOL), big, bound=np.array([1.0]))


def test_check_selection_rounding_bound():
    """The rounding-bound selection check on a hand-made row (ids 0..5, K = 3,
    exact top-3 = {0, 1, 2}, theta = I[2] = 0.004): a swap of the K-th key
    with the next one (gap 0.003) passes exactly when the two keys' bounds
    cover the gap, gamma*(B[3] + B[2]) >= 0.003, and fails otherwise; a key
    far below theta never passes; the relative check rejects the swap, since
    0.003 > 1e-3 * |theta|; a zero bound accepts only the exact top-K."""
    g = check.GAMMA
    I = np.array([5.0, 2.0, 0.004, 0.001, -1.0, -3.0])
    theta = 0.004
    exact = np.array([2, 0, 1])
    swap = np.array([0, 1, 3])
    far = np.array([0, 1, 4])
    wide = np.full(6, 0.003 / (2 * g) * 1.01)     # bounds just cover the gap
    narrow = np.full(6, 0.003 / (2 * g) * 0.99)   # just do not
    zero = np.zeros(6)
    assert check.check_selection_rounding(exact, I, 0, 6, 3, theta, zero) == 0
    assert check.check_selection_rounding(exact, I, 0, 6, 3, theta, narrow) == 0
    assert check.check_selection_rounding(swap, I, 0, 6, 3, theta, wide) == 1
    for bad, B in ((swap, narrow), (swap, zero), (far, wide)):
        with pytest.raises(check.CheckError):
            check.check_selection_rounding(bad, I, 0, 6, 3, theta, B)
    with pytest.raises(check.CheckError):
        check.check_selection(swap, I, 0, 6, 3, theta)
    # only the two keys' own bounds count: a large bound elsewhere changes nothing
    lopsided = narrow.copy()
    lopsided[5] = 1e9
    with pytest.raises(check.CheckError):
        check.check_selection_rounding(swap, I, 0, 6, 3, theta, lopsided)
    # structure is still enforced
    with pytest.raises(check.CheckError):
        check.check_selection_rounding(np.array([0, 0, 1]), I, 0, 6, 3, theta, wide)
