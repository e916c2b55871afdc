"""The fused score kernel's bounded wait, forced from the host.

A finalizing work-group waits for the other chunks' statistics of its
unit.  That wait ends by construction; its bound only keeps a broken
invariant from hanging the GPU.  tri_debug_set_wait_limit(0) makes every
finalizer give up on a slot still unpublished at its second look, so the
outcome tri_score documents for a reached bound can be checked while every
kernel exits normally: raw scores unchanged, heads given up on read
(NaN, 0) in head_stats and drop out of the group maximum (-inf where all
of them do), every other statistic bit-identical, the call's status word
raised (tri_score_status), and the default bound restoring exact results
and a clear status on the next call.
"""
import numpy as np
import pytest
import torch

import rope_aware_key_amd as R
import synth
from harness import gpu_run, units_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_forced_wait_bound_outcome():
    # 16 units of 43 chunks, one chunk per work-group: finalizers run while
    # other chunks of their unit are still streaming
    case = synth.workload_case("long_reasoning", device=DEV, S=2, L=2, n=32768, B=2048)
    ref = gpu_run(case, raw=True, stats=True, compact=False)
    assert R.tri_score_status(ref["workspace"]) == 0
    prev = R.tri_debug_set_wait_limit(0)
    try:
        res = gpu_run(case, raw=True, stats=True, compact=False)
    finally:
        R.tri_debug_set_wait_limit(prev)
    assert prev == 1 << 22
    # the call reports the wait it gave up (the status word of its workspace)
    assert R.tri_score_status(res["workspace"]) == R.TRI_SCORE_WAIT_GAVE_UP
    again = gpu_run(case, raw=True, stats=True, compact=False)
    assert R.tri_score_status(again["workspace"]) == 0
    for key in ("scores", "raw", "head_stats"):
        assert torch.equal(again[key], ref[key]), key

    assert torch.equal(res["raw"], ref["raw"])
    hs, hs_ref = res["head_stats"].cpu().numpy(), ref["head_stats"].cpu().numpy()
    given_up = np.isnan(hs[..., 0])
    assert np.all(hs[..., 1][given_up] == 0.0)
    np.testing.assert_array_equal(hs[~given_up], hs_ref[~given_up])

    # each score: -inf, or the z-score of one of the group's heads, no
    # larger than the exact score (a maximum over fewer heads)
    sc, sc_ref = res["scores"].cpu().numpy(), ref["scores"].cpu().numpy()
    raw = ref["raw"].cpu().numpy().astype(np.float64)
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    n_inf = n_less = 0
    for (s, l, g) in units_of(case):
        start, n = case.unit_rows(s, l, g)
        u = (s * L + l) * H + g
        mu, sigma = hs_ref[u, :, 0], hs_ref[u, :, 1]
        zm = (1.0 / sigma).astype(np.float32).astype(np.float64)
        za = (-mu / sigma).astype(np.float32).astype(np.float64)
        z = raw[start:start + n] * zm + za                      # [n, G]
        got, want = sc[start:start + n].astype(np.float64), sc_ref[start:start + n]
        fin = np.isfinite(got)
        n_inf += int((~fin).sum())
        assert np.all(got[~fin] == -np.inf)
        tol = 1e-5 * np.maximum(1.0, np.abs(z[fin]))
        assert np.all(np.min(np.abs(z[fin] - got[fin, None]) - tol, axis=1) <= 0.0)
        assert np.all(got[fin] <= want[fin] + 1e-5 * np.maximum(1.0, np.abs(want[fin])))
        n_less += int((got[fin] < want[fin]).sum())
    print(f"heads given up on in head_stats: {int(given_up.sum())} of {given_up.size}; "
          f"scores -inf: {n_inf}, below the exact maximum: {n_less}", flush=True)
