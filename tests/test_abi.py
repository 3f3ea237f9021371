"""The C-ABI library loads and exports every entry point include/*.h declares;
host-side argument checks return the documented codes (no GPU needed: these
calls return before any HIP call)."""
import ctypes
import glob
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "scoring_exact_top_amd", "libidxtopk.so")


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b(idx_topk_[a-z_]+)\s*\(",
                             src, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libidxtopk.so not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"idx_topk_prefill", "idx_topk_decode_paged", "idx_topk_prefill_workspace",
            "idx_topk_decode_workspace", "idx_topk_prefill_debug", "idx_topk_read_stats",
            "idx_topk_strerror"} <= names
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_generators():
    src = open(os.path.join(ROOT, "include", "idx_topk.h")).read()
    stride = int(re.search(r"#define IDX_TOPK_SAMPLE_STRIDE (\d+)", src).group(1))
    off = int(re.search(r"#define IDX_TOPK_SAMPLE_OFFSET (\d+)", src).group(1))
    assert (stride, off) == (synth.SAMPLE_STRIDE, synth.SAMPLE_OFFSET)


def test_workspace_queries(lib):
    lib.idx_topk_prefill_workspace.restype = ctypes.c_size_t
    lib.idx_topk_decode_workspace.restype = ctypes.c_size_t
    a = lib.idx_topk_prefill_workspace(64, 8192, 2048)
    b = lib.idx_topk_prefill_workspace(4096, 131072, 2048)
    assert 0 < a < b < (1 << 31)
    assert lib.idx_topk_prefill_workspace(64, 8192, 0) == 0
    assert lib.idx_topk_prefill_workspace(64, 8192, 2049) == 0
    assert lib.idx_topk_decode_workspace(16, 1024, 64, 2048) > 0
    assert lib.idx_topk_decode_workspace(16, 1024, 32, 2048) == 0


def test_host_argument_errors(lib):
    vp = ctypes.c_void_p
    f = lib.idx_topk_prefill
    f.restype = ctypes.c_int
    f.argtypes = [vp] * 7 + [ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_size_t, vp]
    good = vp(1 << 20)          # never dereferenced: every case fails before any launch
    bad_align = vp((1 << 20) + 8)
    ws = vp(1 << 30)
    big = 1 << 40
    args = lambda **kw: [kw.get("q", good), None, kw.get("k", good), good, good, good, good,
                         kw.get("K", 2048), good, kw.get("Q", 4), kw.get("N", 100),
                         kw.get("ws", ws), kw.get("wsb", big), None]
    assert f(*args(K=0)) == -1
    assert f(*args(K=2049)) == -1
    assert f(*args(Q=-1)) == -1
    assert f(*args(q=None)) == -1
    assert f(*args(q=bad_align)) == -1
    assert f(*args(k=bad_align)) == -1
    assert f(*args(ws=None)) == -3
    assert f(*args(wsb=16)) == -3
    assert f(*args(ws=vp((1 << 30) + 64))) == -1     # workspace not 256-byte aligned
    assert f(*args(Q=0)) == 0                         # empty batch: nothing to do
    assert f(*args(N=(1 << 24) - 63)) == -2           # relaid keys past 31-bit offsets
    d = lib.idx_topk_decode_paged
    d.restype = ctypes.c_int
    d.argtypes = [vp] * 7 + [ctypes.c_int32] * 5 + [vp, vp, ctypes.c_size_t, vp]
    dargs = lambda ps=64, K=2048, B=2: [good] * 7 + [B, 8, ps, 16, K, good, ws, big, None]
    assert d(*dargs(ps=32)) == -2
    assert d(*dargs(K=0)) == -1
    assert d(*dargs(B=0)) == 0
    assert d(*dargs(B=65536)) == -2                   # sequences index a grid dimension of 65535
    lib.idx_topk_strerror.restype = ctypes.c_char_p
    assert lib.idx_topk_strerror(-3) == b"workspace missing or too small"


def test_unfused_and_rows_argument_errors(lib):
    vp = ctypes.c_void_p
    lib.idx_topk_prefill_unfused_workspace.restype = ctypes.c_size_t
    fused = lib.idx_topk_prefill_workspace(4096, 131072, 2048)
    unf = lib.idx_topk_prefill_unfused_workspace(4096, 131072, 2048)
    assert unf >= fused + 4096 * 131072 * 4        # plus the dense score matrix
    assert lib.idx_topk_prefill_unfused_workspace(4, 100, 0) == 0
    r = lib.idx_topk_rows
    r.restype = ctypes.c_int
    r.argtypes = [vp, ctypes.c_int64, vp, vp, ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32, vp]
    good = vp(1 << 20)
    rargs = lambda **kw: [kw.get("s", good), kw.get("ld", 100), good, good, kw.get("K", 64), good,
                          kw.get("Q", 4), kw.get("N", 100), None]
    assert r(*rargs(K=0)) == -1
    assert r(*rargs(K=2049)) == -1
    assert r(*rargs(ld=99)) == -1                     # row stride below N
    assert r(*rargs(s=vp((1 << 20) + 4))) == -1       # scores not 16-byte aligned
    assert r(*rargs(s=None)) == -1
    assert r(*rargs(N=1 << 30, ld=1 << 30)) == -2     # rows longer than a buffer resource reaches
    assert r(*rargs(Q=0)) == 0


def test_scan_argument_errors(lib):
    """Argument checks of the BF16 scan and the floor kernel, all answered
    before any device work."""
    vp = ctypes.c_void_p
    f = lib.idx_topk_scan_bf16
    f.restype = ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, ctypes.c_size_t, vp, vp]
    lib.idx_topk_scan_bf16_workspace.restype = ctypes.c_size_t
    lib.idx_topk_scan_bf16_workspace.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    good, ws = vp(1 << 20), vp(1 << 30)
    need = lib.idx_topk_scan_bf16_workspace(32, 262144, 2048)
    assert need >= 32 * 262144 * 4                    # the score rows
    assert lib.idx_topk_scan_bf16_workspace(4, 100, 0) == 0
    args = lambda **kw: [kw.get("q", good), good, kw.get("k", good), good, kw.get("B", 32),
                         kw.get("N", 262144), kw.get("K", 2048), good, kw.get("ws", ws),
                         kw.get("wsb", need), None, None]
    assert f(*args(K=0)) == -1
    assert f(*args(K=2049)) == -1
    assert f(*args(B=-1)) == -1
    assert f(*args(B=65536)) == -2                    # streams index a grid dimension of 65535
    assert f(*args(N=1 << 23)) == -2                  # a stream's keys past a buffer resource's reach
    assert f(*args(q=vp((1 << 20) + 8))) == -1        # q not 16-byte aligned
    assert f(*args(k=None)) == -1
    assert f(*args(ws=None)) == -3
    assert f(*args(wsb=need - 1)) == -3
    assert f(*args(B=0)) == 0
    g = lib.idx_topk_stream_floor
    g.restype = ctypes.c_int
    g.argtypes = [vp, ctypes.c_int64, vp, vp]
    assert g(good, -1, good, None) == -1
    assert g(vp((1 << 20) + 4), 10, good, None) == -1
    assert g(good, 0, good, None) == 0


def test_key_count_limit_is_exact(lib):
    """The largest accepted N is the one whose relaid tiles plus one tile of
    slack stay below 2^31 bytes: (N + 64) * 128 <= 2^31 - 1.  N at the limit
    passes the geometry check (and fails on the missing workspace next), one
    more is unsupported."""
    vp = ctypes.c_void_p
    f = lib.idx_topk_prefill
    f.restype = ctypes.c_int
    f.argtypes = [vp] * 7 + [ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_size_t, vp]
    good = vp(1 << 20)
    n_max = (2 ** 31 - 1) // 128 - 64
    assert n_max == 16777151
    call = lambda N: f(good, None, good, good, good, good, good, 2048, good, 4, N, None, 0, None)
    assert call(n_max) == -3
    assert call(n_max + 1) == -2


def test_debug_knobs_are_rejected_where_they_do_not_apply(lib):
    """row_status, clock_out and math_only belong to the fused prefill: the
    unfused comparator and paged decode reject them; math_only with a forced
    threshold is rejected too.  All answered before any device work."""
    import scoring_exact_top_amd as st
    vp = ctypes.c_void_p
    good, ws, big = vp(1 << 20), vp(1 << 30), 1 << 40
    u = lib.idx_topk_prefill_unfused
    u.restype = ctypes.c_int
    u.argtypes = [vp] * 7 + [ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_size_t, vp,
                             ctypes.POINTER(st.Opts)]
    d = lib.idx_topk_decode_paged_debug
    d.restype = ctypes.c_int
    d.argtypes = [vp] * 7 + [ctypes.c_int32] * 5 + [vp, vp, ctypes.c_size_t, vp, vp, ctypes.POINTER(st.Opts)]
    p = lib.idx_topk_prefill_debug
    p.restype = ctypes.c_int
    p.argtypes = [vp] * 7 + [ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_size_t, vp,
                             vp, vp, ctypes.POINTER(st.Opts)]
    for field, val in (("row_status", good), ("clock_out", good), ("math_only", 1)):
        o = st.Opts()
        setattr(o, field, val)
        assert u(good, None, good, good, good, good, good, 64, good, 4, 100, ws, big, None,
                 ctypes.byref(o)) == -1, field
        assert d(*([good] * 7 + [2, 8, 64, 16, 2048, good, ws, big, None, None]), ctypes.byref(o)) == -1, field
    o = st.Opts()
    o.math_only, o.force_tau = 1, 1
    assert p(good, None, good, good, good, good, good, 64, good, 4, 100, ws, big, None, None, None,
             ctypes.byref(o)) == -1


def test_noalloc_decode_argument_errors(lib):
    """The allocation-free decode answers argument errors like the workspace
    entry point, and a call whose scratch would exceed the static array
    with IDX_ESCRATCH, all before any HIP call."""
    vp = ctypes.c_void_p
    f = lib.idx_topk_decode_paged_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [vp] * 7 + [ctypes.c_int32] * 5 + [vp, vp]
    lib.idx_topk_decode_workspace.restype = ctypes.c_size_t
    good = vp(1 << 20)
    args = lambda B=2, mp=8, ps=64, K=2048: [good] * 7 + [B, mp, ps, 16, K, good, None]
    assert f(*args(ps=32)) == -2
    assert f(*args(K=0)) == -1
    assert f(*args(B=-1)) == -1
    assert f(*args(B=0)) == 0
    limit = 16 << 20
    assert lib.idx_topk_decode_workspace(16, 1024, 64, 2048) <= limit      # the benchmarked batch fits
    assert lib.idx_topk_decode_workspace(64, 1024, 64, 2048) > limit       # this one does not
    assert f(*args(B=64, mp=1024)) == -5
    lib.idx_topk_strerror.restype = ctypes.c_char_p
    assert b"scratch" in lib.idx_topk_strerror(-5)


def test_prefill_walk_geometry():
    """The walk the main kernel takes for Q rows over N keys (host logic, no
    GPU): the geometry of lowest cost in rounds of 512 resident workgroups.
    Rows that fill whole rounds keep one split (1024 rows) or the shared
    walk (4096); odd counts take more splits so that the last round is not
    mostly empty (1200 rows: four splits, 2400 workgroups); 3072 rows avoid
    the shared walk, whose 384 or 768 workgroups would leave a round part
    empty; short rows spread over more splits (64 rows: eight)."""
    import scoring_exact_top_amd as lib
    want = {(1, 8192): (0, 8, 32), (64, 8192): (0, 8, 32), (256, 163840): (0, 4, 16),
            (512, 163840): (0, 2, 8), (1024, 163840): (0, 1, 4), (1200, 131072): (0, 4, 16),
            (2048, 131072): (1, 2, 2), (2560, 131072): (0, 2, 8), (3072, 131072): (0, 1, 4),
            (4093, 20000): (1, 1, 1), (4096, 131072): (1, 1, 1), (5120, 131072): (0, 1, 4),
            (6144, 131072): (1, 2, 2), (8192, 131072): (1, 1, 1)}
    for (Q, N), g in want.items():
        assert lib.prefill_geometry(Q, N) == g, (Q, N, lib.prefill_geometry(Q, N), g)
    for bad in ((-1, 8), (8, -1)):
        with pytest.raises(lib.IdxTopkError):
            lib.prefill_geometry(*bad)
