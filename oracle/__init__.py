"""CPU oracle for the DSA Lightning Indexer with exact top-K.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and bench.py's cpu_baseline
leg are the only users.  The product path (scoring_exact_top_amd) never imports
this package.  The arithmetic lives in idx_oracle.c (plain C, fp64, OpenMP over
rows); this module only builds it with gcc and marshals numpy arrays.

Definitions followed (Fusing Indexer Scoring and Exact Top-k page): the score equation of "1.1
The problem", the inputs/outputs of "2.3 Problem definition" (FP8 Q and KV
"each with scales", head weights, half-open valid range, K int32 indices,
unsorted), and the exactness criterion of the same section.  The paged decode
variant follows the contest report page (arXiv 2608.14560), "DSA TopK Indexer".  The BF16
stream scan follows the page "Deleting the key transpose puts the DSA indexer scan on its
streaming floor" (unquantised BF16 keys per stream, exact top-2048).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "idx_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)


def build() -> str:
    """Compile idx_oracle.c into liboracle.so (always recompiles)."""
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_SO)
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
        lib.oracle_dot_raw.restype = ctypes.c_double
        lib.oracle_dot_raw.argtypes = [_u8p, _u8p]
        lib.oracle_prefill_rows.restype = ctypes.c_int
        lib.oracle_prefill_rows.argtypes = [
            _u8p, _f32p, _u8p, _f32p, _f32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, _i32p, ctypes.c_int32, _f64p, _i32p, _f64p, ctypes.c_int]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [
            _u8p, _f32p, _u8p, _f32p, _f32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _f64p, ctypes.c_int32, _i32p, _f64p,
            ctypes.c_int]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_int]
        lib.oracle_scan_bf16.restype = ctypes.c_int
        lib.oracle_scan_bf16.argtypes = [
            _u16p, _f32p, _u16p, _i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _f64p, _i32p,
            _f64p, ctypes.c_int]
        lib.oracle_topk_of_scores.restype = ctypes.c_int
        lib.oracle_topk_of_scores.argtypes = [_f64p, ctypes.c_int32, ctypes.c_int32, _i32p, _f64p]
        _lib = lib
        return lib


def _p(a, t):
    if a is None:
        return None
    return a.ctypes.data_as(t)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def dot_raw(a8: np.ndarray, b8: np.ndarray) -> float:
    a8 = _c(a8, np.uint8)
    b8 = _c(b8, np.uint8)
    assert a8.size == 128 and b8.size == 128
    return _load().oracle_dot_raw(_p(a8, _u8p), _p(b8, _u8p))


def prefill_rows(q8, q_scale, k8, k_scale, w, row_start, row_end, K, rows=None,
                 want_scores=True, nthreads=0):
    """Oracle top-K (and optionally full score rows) for a subset of rows.

    Returns (topk int32 [n,K], theta float64 [n], scores float64 [n,N] or None).
    """
    lib = _load()
    q8 = _c(q8, np.uint8)
    k8 = _c(k8, np.uint8)
    qs = _c(q_scale, np.float32)
    ks = _c(k_scale, np.float32)
    w = _c(w, np.float32)
    rs = _c(row_start, np.int32)
    re = _c(row_end, np.int32)
    Q, N = int(q8.shape[0]), int(k8.shape[0])
    rows_a = np.arange(Q, dtype=np.int32) if rows is None else _c(rows, np.int32)
    n = int(rows_a.size)
    topk = np.empty((n, K), dtype=np.int32)
    theta = np.empty(n, dtype=np.float64)
    scores = np.empty((n, N), dtype=np.float64) if want_scores else None
    rc = lib.oracle_prefill_rows(_p(q8, _u8p), _p(qs, _f32p), _p(k8, _u8p), _p(ks, _f32p),
                                 _p(w, _f32p), _p(rs, _i32p), _p(re, _i32p), Q, N, int(K),
                                 _p(rows_a, _i32p), n, _p(scores, _f64p), _p(topk, _i32p),
                                 _p(theta, _f64p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_prefill_rows failed: %d" % rc)
    return topk, theta, scores


def prefill_case(case, rows=None, want_scores=True, nthreads=0):
    return prefill_rows(case.q8, case.q_scale, case.k8, case.k_scale, case.w, case.row_start,
                        case.row_end, case.K, rows=rows, want_scores=want_scores,
                        nthreads=nthreads)


def decode_case(case, want_scores=True, nthreads=0):
    """Oracle for a paged decode case: (topk physical ids [B,K], theta [B],
    logical scores [B,max_len] or None)."""
    lib = _load()
    q8 = _c(case.q8, np.uint8)
    qs = _c(case.q_scale, np.float32)
    kc = _c(case.k_cache, np.uint8)
    ks = _c(case.k_scale, np.float32)
    w = _c(case.w, np.float32)
    pt = _c(case.page_table, np.int32)
    sl = _c(case.seq_lens, np.int32)
    B = int(q8.shape[0])
    max_len = int(max(1, sl.max())) if B else 1
    topk = np.empty((B, case.K), dtype=np.int32)
    theta = np.empty(B, dtype=np.float64)
    scores = np.empty((B, max_len), dtype=np.float64) if want_scores else None
    rc = lib.oracle_decode(_p(q8, _u8p), _p(qs, _f32p), _p(kc, _u8p), _p(ks, _f32p), _p(w, _f32p),
                           _p(pt, _i32p), _p(sl, _i32p), B, int(pt.shape[1]), int(case.page_size),
                           int(kc.shape[0]), int(case.K), _p(scores, _f64p), max_len,
                           _p(topk, _i32p), _p(theta, _f64p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_decode failed: %d" % rc)
    return topk, theta, scores


def topk_of_scores(scores, K):
    """Exact top-K positions of an arbitrary score vector (desc, index asc)."""
    lib = _load()
    s = _c(scores, np.float64)
    out = np.empty(K, dtype=np.int32)
    th = np.empty(1, dtype=np.float64)
    rc = lib.oracle_topk_of_scores(_p(s, _f64p), int(s.size), int(K), _p(out, _i32p),
                                   _p(th, _f64p))
    if rc != 0:
        raise ValueError("oracle_topk_of_scores failed")
    return out, float(th[0])


def bf16_value(bits: int) -> float:
    return float(_load().oracle_bf16_value(int(bits)))


def scan_bf16(q16, w, k16, lens, K, want_scores=True, nthreads=0):
    """BF16 stream scan: q16 [B,64,128] uint16, w [B,64] f32, k16 [B,N,128]
    uint16, lens [B] int32.  Returns (topk [B,K] positions, theta [B],
    scores [B,N] or None)."""
    lib = _load()
    q16 = _c(q16, np.uint16)
    k16 = _c(k16, np.uint16)
    w = _c(w, np.float32)
    lens = _c(lens, np.int32)
    B, N = int(k16.shape[0]), int(k16.shape[1])
    topk = np.empty((B, K), dtype=np.int32)
    theta = np.empty(B, dtype=np.float64)
    scores = np.empty((B, N), dtype=np.float64) if want_scores else None
    rc = lib.oracle_scan_bf16(_p(q16, _u16p), _p(w, _f32p), _p(k16, _u16p), _p(lens, _i32p), B, N,
                              int(K), _p(scores, _f64p) if want_scores else None, _p(topk, _i32p),
                              _p(theta, _f64p), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_scan_bf16 failed: %d" % rc)
    return topk, theta, scores
