"""tri_score_noalloc, the entry point for callers that cannot allocate,
against tri_score on the same inputs: the same kernels run on the library's
device scratch instead of a caller workspace, so scores, raw scores and head
statistics must agree bit for bit.  Two calls in a row, the second smaller,
also show that nothing the first call left in the shared scratch reaches
the second."""
import numpy as np
import pytest
import torch

import synth
from harness import pinned, shape_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _score_both(case, raw):
    import rope_aware_key_amd as R
    sh = shape_of(case)
    G = case.shape.group
    rows = case.total_rows()
    cu = pinned(case.cu_len, np.int64)
    cp = pinned(case.cur_pos, np.int32)
    ws = torch.empty(max(R.tri_workspace_bytes(sh, cu), 1), dtype=torch.uint8, device=DEV)
    out = []
    for noalloc in (False, True):
        scores = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
        raw_t = torch.full((rows, G), float("nan"), dtype=torch.float32, device=DEV) if raw else None
        hs = torch.full((case.num_units, G, 2), float("nan"), dtype=torch.float64, device=DEV)
        args = (sh, cu, cp, case.k, case.k_pos, case.q_centre, case.q_absmean, case.q_R, scores)
        if noalloc:
            R.tri_score_noalloc(*args, raw_scores=raw_t, head_stats=hs)
        else:
            R.tri_score(*args, raw_scores=raw_t, head_stats=hs, workspace=ws)
        torch.cuda.synchronize()
        out.append((scores.cpu().numpy(), None if raw_t is None else raw_t.cpu().numpy(),
                    hs.cpu().numpy()))
    return out


@pytest.mark.parametrize("raw", [False, True])
def test_noalloc_matches_tri_score_on_two_calls(raw):
    shape = synth.Shape(128, 28, 4, 2)   # GQA group 7, two layers
    big = synth.build_case("noalloc_big", shape, [5000, 3001], [512, 256], device=DEV, seed=5)
    small = synth.build_case("noalloc_small", shape, [700], [128], device=DEV, seed=6)
    for case in (big, small):
        print(f"case {case.cu_len.tolist()} raw={raw}", flush=True)
        (s0, r0, h0), (s1, r1, h1) = _score_both(case, raw)
        assert np.isfinite(s0).all()
        np.testing.assert_array_equal(s1, s0)
        if raw:
            np.testing.assert_array_equal(r1, r0)
        np.testing.assert_array_equal(h1, h0)
