"""The allocation-free paged decode (idx_topk_decode_paged_noalloc) against
the workspace entry point on the same inputs: identical output, on two calls
in a row through the C ABI, the second with a smaller batch (the static
scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _dev(case):
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return [t(case.q8), t(case.q_scale), t(case.k_cache), t(case.k_scale), t(case.w), t(case.page_table),
            t(case.seq_lens)]


def _both(lib, case):
    d = _dev(case)
    ws = lib.alloc_workspace(lib.decode_workspace_bytes(case.B, case.max_pages, case.page_size, case.K), "cuda")
    ref = lib.decode_paged(*d, case.K, workspace=ws)
    out = torch.full((case.B, case.K), -7, dtype=torch.int32, device="cuda")
    lib.decode_paged_noalloc(*d, case.K, out)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


def test_noalloc_decode_matches_the_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import scoring_exact_top_amd as lib
    big = synth.paged_decode(0)                         # the benchmarked batch: 16 sequences
    small = synth.decode_case("noalloc_small", [3000, 100, 2049, 9000, 1], seed=41, max_pages=200)
    for case in (big, small):
        need = lib.decode_workspace_bytes(case.B, case.max_pages, case.page_size, case.K)
        assert need <= lib.NOALLOC_SCRATCH_BYTES
        ref, out = _both(lib, case)
        print(case.name, "B", case.B, "scratch bytes", need, flush=True)
        # index work: bit-exact, row by row (the lowest-position tie rule makes each row's set
        # unique; the order inside a row is not part of the contract)
        assert np.array_equal(np.sort(ref, axis=1), np.sort(out, axis=1)), case.name
