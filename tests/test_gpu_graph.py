"""Graph capture of the multi-kernel calls (idx_topk_graph_*): every replay
equals the eager call on the same inputs, with eager work and
synchronisations between the replays; replays see new data written into the
recorded input buffers; one graph can hold several calls."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

from gpu_util import dev_prefill, log  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import scoring_exact_top_amd  # noqa: F401


def _sorted(x):
    return torch.sort(x, dim=1).values.cpu()


def _prefill_call(lib, d, K, out, ws):
    return lambda: lib.prefill(d["q8"], d["q_scale"], d["k8"], d["k_scale"], d["w"], d["row_start"],
                               d["row_end"], K, out=out, workspace=ws)


def test_graph_prefill_replays():
    import scoring_exact_top_amd as lib
    case = synth.prefill_smoke(0)
    log("case", case.name)
    d = dev_prefill(case)
    nb = lib.prefill_workspace_bytes(case.Q, case.N, case.K)
    ws_e, ws_g = lib.alloc_workspace(nb, "cuda"), lib.alloc_workspace(nb, "cuda")
    out_e = torch.empty((case.Q, case.K), dtype=torch.int32, device="cuda")
    out_g = torch.empty_like(out_e)
    eager = _prefill_call(lib, d, case.K, out_e, ws_e)
    eager()
    torch.cuda.synchronize()
    want = _sorted(out_e)
    g = lib.capture(_prefill_call(lib, d, case.K, out_g, ws_g))
    for rep in range(4):
        out_g.fill_(-7)
        eager()  # the program's own work between replays
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(_sorted(out_g), want), "replay %d differs from the eager call" % rep
        assert lib.read_stats(ws_g)["rows"] == case.Q
    # new data in the recorded buffers: the replay computes on it
    other = synth.prefill_smoke(1)
    d2 = dev_prefill(other)
    for k in ("q8", "k8", "k_scale", "w"):
        d[k].copy_(d2[k])
    if d["q_scale"] is not None:
        d["q_scale"].copy_(d2["q_scale"])
    eager()
    torch.cuda.synchronize()
    want2 = _sorted(out_e)
    assert not torch.equal(want2, want)
    out_g.fill_(-7)
    g.launch()
    torch.cuda.synchronize()
    assert torch.equal(_sorted(out_g), want2)
    g.destroy()


def test_graph_decode_and_scan_in_one_graph():
    import scoring_exact_top_amd as lib
    dc = synth.paged_decode(0)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dd = {k: t(getattr(dc, k)) for k in ("q8", "q_scale", "k_cache", "k_scale", "w", "page_table", "seq_lens")}
    sc = synth.scan_case("graph_scan", 6, 20000, seed=3, lens=[20000, 0, 1500, 19999, 4097, 20000])
    q16, k16 = t(sc.q16.view(np.int16)), t(sc.k16.view(np.int16))
    w16, lens = t(sc.w), t(sc.lens)
    dnb = lib.decode_workspace_bytes(dc.B, dc.max_pages, dc.page_size, dc.K)
    snb = lib.scan_bf16_workspace_bytes(sc.B, sc.N, sc.K)
    dws_e, dws_g = lib.alloc_workspace(dnb, "cuda"), lib.alloc_workspace(dnb, "cuda")
    sws_e, sws_g = lib.alloc_workspace(snb, "cuda"), lib.alloc_workspace(snb, "cuda")
    dout_e = torch.empty((dc.B, dc.K), dtype=torch.int32, device="cuda")
    dout_g = torch.empty_like(dout_e)
    sout_e = torch.empty((sc.B, sc.K), dtype=torch.int32, device="cuda")
    sout_g = torch.empty_like(sout_e)

    def calls(dout, dws, sout, sws):
        lib.decode_paged(dd["q8"], dd["q_scale"], dd["k_cache"], dd["k_scale"], dd["w"], dd["page_table"],
                         dd["seq_lens"], dc.K, out=dout, workspace=dws)
        lib.scan_bf16(q16, w16, k16, lens, sc.K, out=sout, workspace=sws)

    calls(dout_e, dws_e, sout_e, sws_e)
    torch.cuda.synchronize()
    dwant, swant = _sorted(dout_e), _sorted(sout_e)
    g = lib.capture(lambda: calls(dout_g, dws_g, sout_g, sws_g))
    for rep in range(3):
        dout_g.fill_(-7)
        sout_g.fill_(-7)
        calls(dout_e, dws_e, sout_e, sws_e)
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(_sorted(dout_g), dwant), "decode, replay %d" % rep
        assert torch.equal(_sorted(sout_g), swant), "scan, replay %d" % rep
    g.destroy()


def test_graph_capture_errors():
    """A failing call inside the capture ends it (the stream is usable again)
    and raises; the NULL stream cannot be captured."""
    import scoring_exact_top_amd as lib
    raw = lib.raw_library()
    assert raw.idx_topk_graph_begin(None) != 0
    assert raw.idx_topk_graph_launch(None, None) != 0
    assert raw.idx_topk_graph_destroy(None) == 0
    case = synth.prefill_smoke(0)
    d = dev_prefill(case)
    out = torch.empty((case.Q, case.K), dtype=torch.int32, device="cuda")
    small = lib.alloc_workspace(256, "cuda")  # too small: the call fails inside the capture
    s = torch.cuda.Stream()
    with pytest.raises(Exception):
        lib.capture(_prefill_call(lib, d, case.K, out, small), stream=s)
    # the stream works normally afterwards
    ws = lib.alloc_workspace(lib.prefill_workspace_bytes(case.Q, case.N, case.K), "cuda")
    with torch.cuda.stream(s):
        _prefill_call(lib, d, case.K, out, ws)()
    s.synchronize()
    assert (out.cpu().numpy()[:, 0] >= 0).all()
