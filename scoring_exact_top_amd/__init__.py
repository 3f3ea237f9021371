"""DSA Lightning Indexer scoring fused with exact top-K on MI355X (gfx950).

Thin ctypes binding of libidxtopk.so (C ABI in include/idx_topk.h).  This
module only marshals arguments: torch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
Importing raises if the library has not been built (run
``python scoring_exact_top_amd/build.py`` or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libidxtopk.so")

HEADS = 64
DIM = 128
KMAX = 2048
PAGE = 64

if not os.path.exists(LIB_PATH):
    raise ImportError("libidxtopk.so is not built at %s; run python scoring_exact_top_amd/build.py"
                      % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class Opts(ctypes.Structure):
    _fields_ = [("force_tau", ctypes.c_int32), ("tau_value", ctypes.c_float),
                ("cand_cap", ctypes.c_int32),
                ("ev_main_start", ctypes.c_void_p), ("ev_main_stop", ctypes.c_void_p),
                ("main_reps", ctypes.c_int32), ("row_status", ctypes.c_void_p),
                ("clock_out", ctypes.c_void_p), ("math_only", ctypes.c_int32)]


# Row outcomes written to row_status (idx_topk.h IDX_ROW_*).
ROW_FAST, ROW_UNDERFLOW, ROW_OVERFLOW, ROW_BAD = 0, 1, 2, -1


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in
                ("rows", "fast_ok", "underflow", "overflow", "many_cands", "repaired", "trivial",
                 "bad_rows")]

    def asdict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_lib.idx_topk_prefill_workspace.restype = _sz
_lib.idx_topk_prefill_workspace.argtypes = [_i32, _i32, _i32]
_lib.idx_topk_prefill_geometry.restype = _i32
_lib.idx_topk_prefill_geometry.argtypes = [_i32, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
_lib.idx_topk_prefill.restype = ctypes.c_int
_lib.idx_topk_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _vp, _sz,
                                  _vp]
_lib.idx_topk_prefill_debug.restype = ctypes.c_int
_lib.idx_topk_prefill_debug.argtypes = _lib.idx_topk_prefill.argtypes + [_vp, _vp,
                                                                          ctypes.POINTER(Opts)]
_lib.idx_topk_prefill_unfused_workspace.restype = _sz
_lib.idx_topk_prefill_unfused_workspace.argtypes = [_i32, _i32, _i32]
_lib.idx_topk_prefill_unfused.restype = ctypes.c_int
_lib.idx_topk_prefill_unfused.argtypes = _lib.idx_topk_prefill.argtypes + [ctypes.POINTER(Opts)]
_lib.idx_topk_rows.restype = ctypes.c_int
_lib.idx_topk_rows.argtypes = [_vp, ctypes.c_int64, _vp, _vp, _i32, _vp, _i32, _i32, _vp]
_lib.idx_topk_scan_bf16_workspace.restype = _sz
_lib.idx_topk_scan_bf16_workspace.argtypes = [_i32, _i32, _i32]
_lib.idx_topk_scan_bf16.restype = ctypes.c_int
_lib.idx_topk_scan_bf16.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp,
                                    ctypes.POINTER(Opts)]
_lib.idx_topk_scan_bf16_scores.restype = ctypes.c_void_p
_lib.idx_topk_scan_bf16_scores.argtypes = [_vp, _i32, _i32]
_lib.idx_topk_stream_floor.restype = ctypes.c_int
_lib.idx_topk_stream_floor.argtypes = [_vp, ctypes.c_int64, _vp, _vp]
_lib.idx_topk_decode_workspace.restype = _sz
_lib.idx_topk_decode_workspace.argtypes = [_i32, _i32, _i32, _i32]
_lib.idx_topk_decode_paged.restype = ctypes.c_int
_lib.idx_topk_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                       _i32, _vp, _vp, _sz, _vp]
_lib.idx_topk_decode_paged_debug.restype = ctypes.c_int
_lib.idx_topk_decode_paged_debug.argtypes = _lib.idx_topk_decode_paged.argtypes + [_vp, ctypes.POINTER(Opts)]
_lib.idx_topk_decode_paged_noalloc.restype = ctypes.c_int
_lib.idx_topk_decode_paged_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp]
_lib.idx_topk_read_stats.restype = ctypes.c_int
_lib.idx_topk_read_stats.argtypes = [_vp, ctypes.POINTER(Stats), _vp]
_lib.idx_topk_strerror.restype = ctypes.c_char_p
_lib.idx_topk_strerror.argtypes = [ctypes.c_int]


class IdxTopkError(RuntimeError):
    def __init__(self, code: int):
        super().__init__("idx_topk error %d: %s" % (code, _lib.idx_topk_strerror(code).decode()))
        self.code = code


def _check(rc: int):
    if rc != 0:
        raise IdxTopkError(rc)


def _ptr(t: Optional[torch.Tensor], dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError("expected dtype %s, got %s" % (dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def prefill_workspace_bytes(Q: int, N: int, K: int) -> int:
    return int(_lib.idx_topk_prefill_workspace(Q, N, K))


def prefill_geometry(Q: int, N: int):
    """(shared, splits, segments) of the main kernel's walk for Q rows over
    N keys; see idx_topk_prefill_geometry in include/idx_topk.h."""
    sh, sp, sg = _i32(), _i32(), _i32()
    _check(_lib.idx_topk_prefill_geometry(Q, N, ctypes.byref(sh), ctypes.byref(sp), ctypes.byref(sg)))
    return int(sh.value), int(sp.value), int(sg.value)


def prefill_unfused_workspace_bytes(Q: int, N: int, K: int) -> int:
    return int(_lib.idx_topk_prefill_unfused_workspace(Q, N, K))


def scan_bf16_workspace_bytes(B: int, N: int, K: int) -> int:
    return int(_lib.idx_topk_scan_bf16_workspace(B, N, K))


def decode_workspace_bytes(B: int, max_pages: int, page_size: int, K: int) -> int:
    return int(_lib.idx_topk_decode_workspace(B, max_pages, page_size, K))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _q_k(q8, k8):
    if q8.dtype == torch.float8_e4m3fn:
        q8 = q8.view(torch.uint8)
    if k8.dtype == torch.float8_e4m3fn:
        k8 = k8.view(torch.uint8)
    return q8, k8


def prefill(q8, q_scale, k8, k_scale, w, row_start, row_end, K: int, out=None, workspace=None,
            stream=None):
    """Top-K key ids per query row; see idx_topk_prefill in include/idx_topk.h.

    q8 [Q,64,128] uint8 (or float8_e4m3fn), q_scale [Q,64] f32 or None,
    k8 [N,128], k_scale [N] f32, w [Q,64] f32, row_start/row_end [Q] int32.
    Returns out [Q,K] int32 (absolute ids, unsorted, -1 padded).
    """
    return _prefill(q8, q_scale, k8, k_scale, w, row_start, row_end, K, out, workspace, stream,
                    debug=False)


def prefill_debug(q8, q_scale, k8, k_scale, w, row_start, row_end, K: int, out=None,
                  workspace=None, stream=None, scores_out=None, tau_out=None,
                  force_tau: Optional[float] = None, cand_cap: int = 0,
                  main_events=None, main_reps: int = 1, row_status=None, clock_out=None,
                  math_only: bool = False):
    """idx_topk_prefill_debug: also emits FP32 scores [Q,N] and thresholds [Q].

    main_events: optional (start, stop) pair of torch.cuda.Event(enable_timing=True)
    recorded around the fused main kernel; main_reps > 1 launches that kernel
    so many times back to back inside the pair (timing only).  row_status [Q]
    int32 receives each row's ROW_* outcome; clock_out [2] int64 (zeroed by
    the caller) accumulates the main kernel's shader-clock cycles and
    wall-clock ticks; math_only runs the control build of the main kernel
    (no selection, out is not written)."""
    ev0 = ev1 = None
    if main_events is not None:
        ev0, ev1 = (ctypes.c_void_p(e.cuda_event) for e in main_events)
    opts = Opts(1 if force_tau is not None else 0, float(force_tau or 0.0), int(cand_cap),
                ev0, ev1, int(main_reps), _ptr(row_status, torch.int32),
                _ptr(clock_out, torch.int64), 1 if math_only else 0)
    return _prefill(q8, q_scale, k8, k_scale, w, row_start, row_end, K, out, workspace, stream,
                    debug=True, scores_out=scores_out, tau_out=tau_out, opts=opts)


def _prefill(q8, q_scale, k8, k_scale, w, row_start, row_end, K, out, workspace, stream, debug,
             scores_out=None, tau_out=None, opts=None):
    q8, k8 = _q_k(q8, k8)
    Q, N = int(q8.shape[0]), int(k8.shape[0])
    if q8.shape[1:] != (HEADS, DIM) or k8.shape[1:] != (DIM,):
        raise ValueError("q8 must be [Q,64,128] and k8 [N,128]")
    dev = q8.device
    if out is None:
        out = torch.empty((Q, K), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(prefill_workspace_bytes(Q, N, K), dev)
    args = [_ptr(q8, torch.uint8), _ptr(q_scale, torch.float32), _ptr(k8, torch.uint8),
            _ptr(k_scale, torch.float32), _ptr(w, torch.float32), _ptr(row_start, torch.int32),
            _ptr(row_end, torch.int32), int(K), _ptr(out, torch.int32), Q, N, _ptr(workspace),
            int(workspace.numel()), _stream(stream)]
    if debug:
        _check(_lib.idx_topk_prefill_debug(*args, _ptr(scores_out, torch.float32),
                                           _ptr(tau_out, torch.float32), ctypes.byref(opts)))
    else:
        _check(_lib.idx_topk_prefill(*args))
    return out


def prefill_unfused(q8, q_scale, k8, k_scale, w, row_start, row_end, K: int, out=None,
                    workspace=None, stream=None, main_events=None, main_reps: int = 1):
    """idx_topk_prefill_unfused: the same scores written to an explicit [Q,N]
    matrix in the workspace, then a separate top-K over it (the comparator of
    the fused path).  main_events: optional (start, stop) event pair around
    the scoring kernel."""
    q8, k8 = _q_k(q8, k8)
    Q, N = int(q8.shape[0]), int(k8.shape[0])
    if q8.shape[1:] != (HEADS, DIM) or k8.shape[1:] != (DIM,):
        raise ValueError("q8 must be [Q,64,128] and k8 [N,128]")
    dev = q8.device
    if out is None:
        out = torch.empty((Q, K), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(prefill_unfused_workspace_bytes(Q, N, K), dev)
    ev0 = ev1 = None
    if main_events is not None:
        ev0, ev1 = (ctypes.c_void_p(e.cuda_event) for e in main_events)
    opts = Opts(0, 0.0, 0, ev0, ev1, int(main_reps))
    _check(_lib.idx_topk_prefill_unfused(
        _ptr(q8, torch.uint8), _ptr(q_scale, torch.float32), _ptr(k8, torch.uint8),
        _ptr(k_scale, torch.float32), _ptr(w, torch.float32), _ptr(row_start, torch.int32),
        _ptr(row_end, torch.int32), int(K), _ptr(out, torch.int32), Q, N, _ptr(workspace),
        int(workspace.numel()), _stream(stream), ctypes.byref(opts)))
    return out


def topk_rows(scores, row_start, row_end, K: int, out=None, stream=None):
    """idx_topk_rows: exact top-K positions of each row of a dense FP32
    matrix scores [Q, ld] over [row_start, row_end) (ties to the lowest
    positions; rows with fewer than K positions are -1 padded)."""
    if scores.dim() != 2:
        raise ValueError("scores must be [Q, N]")
    Q, N = int(scores.shape[0]), int(scores.shape[1])
    if out is None:
        out = torch.empty((Q, K), dtype=torch.int32, device=scores.device)
    _check(_lib.idx_topk_rows(_ptr(scores, torch.float32), N, _ptr(row_start, torch.int32),
                              _ptr(row_end, torch.int32), int(K), _ptr(out, torch.int32), Q, N,
                              _stream(stream)))
    return out


def scan_bf16(q16, w, k16, lens, K: int, out=None, workspace=None, stream=None, main_events=None,
              main_reps: int = 1):
    """idx_topk_scan_bf16: q16 [B,64,128] and k16 [B,N,128] as torch.bfloat16 or
    uint16/int16 bit patterns, w [B,64] f32, lens [B] int32 (device).  Returns
    out [B,K] int32 key positions.  main_events / main_reps: timing of the
    scoring kernel."""
    if q16.dtype == torch.bfloat16:
        q16 = q16.view(torch.int16)
    if k16.dtype == torch.bfloat16:
        k16 = k16.view(torch.int16)
    B, N = int(k16.shape[0]), int(k16.shape[1])
    if q16.shape != (B, HEADS, DIM) or k16.shape[2:] != (DIM,):
        raise ValueError("q16 must be [B,64,128] and k16 [B,N,128]")
    dev = q16.device
    if out is None:
        out = torch.empty((B, K), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(scan_bf16_workspace_bytes(B, N, K), dev)
    ev0 = ev1 = None
    if main_events is not None:
        ev0, ev1 = (ctypes.c_void_p(e.cuda_event) for e in main_events)
    opts = Opts(0, 0.0, 0, ev0, ev1, int(main_reps))
    _check(_lib.idx_topk_scan_bf16(_ptr(q16), _ptr(w, torch.float32), _ptr(k16), _ptr(lens, torch.int32),
                                   B, N, int(K), _ptr(out, torch.int32), _ptr(workspace),
                                   int(workspace.numel()), _stream(stream), ctypes.byref(opts)))
    return out


def scan_bf16_scores(workspace: torch.Tensor, B: int, N: int) -> torch.Tensor:
    """The [B,N] FP32 score rows inside a scan workspace (a copy; tests only)."""
    addr = _lib.idx_topk_scan_bf16_scores(_ptr(workspace), int(B), int(N))
    off = int(addr) - workspace.data_ptr()
    return workspace[off: off + 4 * B * N].view(torch.float32).view(B, N).clone()


_lib.idx_topk_graph_begin.restype = ctypes.c_int
_lib.idx_topk_graph_begin.argtypes = [_vp]
_lib.idx_topk_graph_end.restype = ctypes.c_int
_lib.idx_topk_graph_end.argtypes = [_vp, ctypes.POINTER(_vp)]
_lib.idx_topk_graph_launch.restype = ctypes.c_int
_lib.idx_topk_graph_launch.argtypes = [_vp, _vp]
_lib.idx_topk_graph_destroy.restype = ctypes.c_int
_lib.idx_topk_graph_destroy.argtypes = [_vp]


class Graph:
    """A recorded chain of library calls (idx_topk_graph_*); launch() replays it."""

    def __init__(self, handle):
        self._h = handle

    def launch(self, stream=None):
        if not self._h:
            raise ValueError("graph is destroyed")
        _check(_lib.idx_topk_graph_launch(self._h, _stream(stream)))

    def destroy(self):
        if self._h:
            h, self._h = self._h, None
            _check(_lib.idx_topk_graph_destroy(h))

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def capture(fn, stream=None) -> Graph:
    """Record the library calls that fn() makes into a graph.  fn runs with a
    side stream (or `stream`) current; it must pass its own output and
    workspace buffers (nothing may allocate during the capture) and no
    timing events."""
    s = stream if stream is not None else torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _check(_lib.idx_topk_graph_begin(_stream(s)))
        h = _vp()
        try:
            fn()
        except BaseException:
            _lib.idx_topk_graph_end(_stream(s), ctypes.byref(h))
            if h:
                _lib.idx_topk_graph_destroy(h)
            raise
        _check(_lib.idx_topk_graph_end(_stream(s), ctypes.byref(h)))
    return Graph(h)


def stream_floor(src: torch.Tensor, out=None, stream=None):
    """idx_topk_stream_floor over src viewed as 256-byte records."""
    nbytes = src.numel() * src.element_size()
    n = nbytes // 256
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=src.device)
    _check(_lib.idx_topk_stream_floor(_ptr(src), int(n), _ptr(out, torch.float32), _stream(stream)))
    return out


def decode_paged(q8, q_scale, k_cache, k_scale, w, page_table, seq_lens, K: int, out=None,
                 workspace=None, stream=None, force_tau: Optional[float] = None, main_events=None,
                 main_reps: int = 1, scores_out=None):
    """Top-K physical cache slots per sequence; see idx_topk_decode_paged.

    q8 [B,64,128], q_scale [B,64] or None, k_cache [P,64,128], k_scale [P,64],
    w [B,64], page_table [B,max_pages] int32, seq_lens [B] int32 (device).
    main_events selects idx_topk_decode_paged_debug with a (start, stop)
    torch.cuda.Event pair around the scoring kernel; scores_out
    [B, max_pages*64] f32 (debug entry too) receives the scores the
    selection read; force_tau is passed through so that the library's
    rejection of it (decode has no threshold knob) can be tested.
    """
    q8, k_cache = _q_k(q8, k_cache)
    B = int(q8.shape[0])
    P, page = int(k_cache.shape[0]), int(k_cache.shape[1])
    max_pages = int(page_table.shape[1])
    dev = q8.device
    if out is None:
        out = torch.empty((B, K), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(decode_workspace_bytes(B, max_pages, page, K), dev)
    args = [_ptr(q8, torch.uint8), _ptr(q_scale, torch.float32), _ptr(k_cache, torch.uint8),
            _ptr(k_scale, torch.float32), _ptr(w, torch.float32), _ptr(page_table, torch.int32),
            _ptr(seq_lens, torch.int32), B, max_pages, page, P, int(K), _ptr(out, torch.int32),
            _ptr(workspace), int(workspace.numel()), _stream(stream)]
    if force_tau is None and main_events is None and main_reps == 1 and scores_out is None:
        _check(_lib.idx_topk_decode_paged(*args))
    else:
        ev0 = ev1 = None
        if main_events is not None:
            ev0, ev1 = (ctypes.c_void_p(e.cuda_event) for e in main_events)
        opts = Opts(1 if force_tau is not None else 0, float(force_tau or 0.0), 0, ev0, ev1,
                    int(main_reps))
        _check(_lib.idx_topk_decode_paged_debug(*args, _ptr(scores_out, torch.float32), ctypes.byref(opts)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_paged_noalloc(q8, q_scale, k_cache, k_scale, w, page_table, seq_lens, K: int, out, stream=None):
    """idx_topk_decode_paged_noalloc: paged decode with the library's static
    per-GPU scratch (no workspace, nothing allocated); `out` [B,K] int32 is
    the caller's."""
    q8, k_cache = _q_k(q8, k_cache)
    B = int(q8.shape[0])
    P, page = int(k_cache.shape[0]), int(k_cache.shape[1])
    _check(_lib.idx_topk_decode_paged_noalloc(
        _ptr(q8, torch.uint8), _ptr(q_scale, torch.float32), _ptr(k_cache, torch.uint8),
        _ptr(k_scale, torch.float32), _ptr(w, torch.float32), _ptr(page_table, torch.int32),
        _ptr(seq_lens, torch.int32), B, int(page_table.shape[1]), page, P, int(K), _ptr(out, torch.int32),
        _stream(stream)))
    return out


def read_stats(workspace: torch.Tensor, stream=None) -> dict:
    st = Stats()
    _check(_lib.idx_topk_read_stats(_ptr(workspace), ctypes.byref(st), _stream(stream)))
    return st.asdict()


def raw_library():
    """The loaded ctypes library (for ABI-level tests)."""
    return _lib
