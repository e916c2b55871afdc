"""Parity of tri_score_offsets (offset-set variants) against the fp64 oracle.

The oracle's offset variants are pinned in test_oracle_pins.py (the maximum
over offsets equals the maximum of the exact logits when the queries sit on
their centre; the mean over any set equals the mean logit).  Here the HIP
path is held to the same bars as tri_score:
  scores  |gpu - ref| <= 1e-4 * max(1, |ref|)
  raw     |gpu - ref| <= 1e-4 * max(|ref|, sigma_h)
  mu, sigma within 1e-5 of sigma
and the default set {2^0..2^16} averaged must reproduce tri_score bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import (z_floor, check_raw, check_scores, check_selection_exact, gpu_run, gpu_score_offsets,
                     oracle_unit, units_of)

pytestmark = pytest.mark.gpu

DEV = "cuda"

DEFAULT = [2.0 ** j for j in range(17)]
LINEAR = [float(x) for x in range(1, 129, 8)]          # 16 linearly spaced offsets
SHORT = [2.0 ** j for j in range(9)]                   # maximum distance 256
SINGLE = [0.0]                                         # the current position only
ODD = [0.5, 3.0, 1000.0, -7.0, 65536.0]                # non-integer, negative, far

SETS = {"default": DEFAULT, "linear": LINEAR, "short": SHORT, "single": SINGLE, "odd": ODD}


def _compare(case, res, units, offsets, reduce, factored=True):
    scores = res["scores"].cpu().numpy()
    raw = res["raw"].cpu().numpy() if res.get("raw") is not None else None
    hs = res["head_stats"].cpu().numpy() if res.get("head_stats") is not None else None
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    for (s, l, g) in units:
        if case.seq_len(s) == 0:
            continue
        start, n, ref, S, mu, sigma = oracle_unit(case, s, l, g, factored=factored,
                                                  offsets=offsets, reduce=reduce)
        what = f"{reduce} unit {(s, l, g)}"
        check_scores(scores[start:start + n], ref, what, z_floor(S, sigma))
        if raw is not None:
            check_raw(raw[start:start + n], S, sigma, "raw " + what)
        if hs is not None:
            u = (s * L + l) * H + g
            np.testing.assert_allclose(hs[u, :, 0], mu, rtol=0, atol=1e-5 * max(np.max(sigma), np.max(np.abs(S))))
            np.testing.assert_allclose(hs[u, :, 1], sigma, rtol=1e-5, atol=1e-5 * np.max(np.abs(S)))


def _bits(t):
    return t.view(torch.uint8) if t.dtype.is_floating_point else t


# ------------------------------------------------ mean over the offsets
@pytest.mark.parametrize("d,G", [(128, 7), (48, 3)])
def test_default_set_equals_tri_score_bitwise(d, G):
    """The mean over {2^0..2^16} given explicitly is tri_score itself (fused
    MFMA path at d = 128, generic VALU path at d = 48)."""
    shape = synth.Shape(d, 2 * G, 2, 1)
    case = synth.build_case("dflt", shape, [3000, 1025, 37], [500, 1025, 4], device=DEV, seed=d)
    a = gpu_run(case, compact=False)
    b = gpu_score_offsets(case, DEFAULT, "mean")
    for key in ("scores", "raw", "head_stats"):
        assert torch.equal(_bits(a[key]), _bits(b[key])), key


@pytest.mark.parametrize("name", ["linear", "short", "single", "odd"])
@pytest.mark.parametrize("d,G", [(128, 7), (48, 3)])
def test_mean_over_other_sets(name, d, G):
    shape = synth.Shape(d, 2 * G, 2, 1)
    case = synth.build_case("mean", shape, [2500, 1100, 0, 64], [300, 50, 5, 64], device=DEV,
                            seed=d + len(name))
    res = gpu_score_offsets(case, SETS[name], "mean")
    units = units_of(case)
    _compare(case, res, units, SETS[name], "mean")
    _compare(case, res, units[:1], SETS[name], "mean", factored=False)


# ------------------------------------------------- max over the offsets
@pytest.mark.parametrize("name", list(SETS))
def test_max_long_reasoning_shape(name):
    """G = 7, d = 128 (the long-reasoning shape), 5000 keys: five tickets of
    one unit, the last ragged."""
    case = synth.workload_case("long_reasoning", device=DEV, S=1, L=1, n=5000, B=2048)
    res = gpu_score_offsets(case, SETS[name], "max")
    units = units_of(case)
    _compare(case, res, units, SETS[name], "max")
    _compare(case, res, units[:1], SETS[name], "max", factored=False)


@pytest.mark.parametrize("d,G,offsets", [
    (64, 8, DEFAULT),        # two head rounds of 5 tiles, GB = 4
    (256, 2, DEFAULT),       # eight MFMA steps, GB = 2
    (32, 16, SHORT),         # one step, 16 heads (four rounds) in one pass
    (96, 5, LINEAR),         # three steps, five heads: the second round holds one
    (128, 16, DEFAULT),      # 16 heads of 5 tiles at 12 per pass: two passes
    (256, 8, LINEAR),        # 24 KB tiles, 4 tiles a head: two passes of 4 heads
    (128, 1, [float(x) for x in range(1, 161)]),   # 160 rows: one head over all slots
    (128, 4, [0.5 * x for x in range(100)]),       # spread heads, one per pass: four passes
    (64, 3, [float(x) for x in range(1, 384, 2)]), # spread, 12 tiles a head: passes of 2 + 1 heads
])
def test_max_shapes_and_passes(d, G, offsets):
    shape = synth.Shape(d, 2 * G, 2, 2)
    case = synth.build_case("max", shape, [1500, 2100, 0, 37], [300, 2100, 5, 40], device=DEV,
                            seed=d + G)
    res = gpu_score_offsets(case, offsets, "max")
    units = units_of(case)
    _compare(case, res, units, offsets, "max")
    _compare(case, res, units[-1:], offsets, "max", factored=False)


def test_max_ragged_batch_then_select():
    """Many ragged sequences (tickets of several units share a work-group),
    raw scores spilled to the workspace, then selection and compaction on
    the max-reduced scores."""
    case = synth.workload_case("ragged", device=DEV, S=6, L=1, n_range=(100, 3000))
    res = gpu_score_offsets(case, DEFAULT, "max", raw_in_ws=True)
    units = units_of(case)
    _compare(case, res, units, DEFAULT, "max")
    out = gpu_run(case, scores_in=res["scores"])
    check_selection_exact(case, out)


def test_single_offset_max_equals_mean():
    """With one offset the maximum and the mean are the same score."""
    case = synth.workload_case("long_reasoning", device=DEV, S=1, L=1, n=3000, B=700)
    mx = gpu_score_offsets(case, [1024.0], "max")
    mn = gpu_score_offsets(case, [1024.0], "mean")
    a, b = mx["scores"].cpu().numpy(), mn["scores"].cpu().numpy()
    assert np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) <= 2e-4


def test_max_deterministic_bitwise():
    case = synth.workload_case("long_reasoning", device=DEV, S=1, L=2, n=3000, B=700)
    a = gpu_score_offsets(case, DEFAULT, "max")
    b = gpu_score_offsets(case, DEFAULT, "max")
    for key in ("scores", "raw", "head_stats"):
        assert torch.equal(_bits(a[key]), _bits(b[key])), key


@pytest.mark.timeout(600)
def test_max_long_reasoning_full_size_sampled():
    """32K -> 2048 workload at full size with the maximum over the default
    set: sampled units against the oracle, selection exact on every unit."""
    case = synth.workload_case("long_reasoning", device=DEV)
    res = gpu_score_offsets(case, DEFAULT, "max", raw=False)
    units = units_of(case)
    g = np.random.default_rng(9)
    samp = [units[i] for i in sorted(g.choice(len(units), size=4, replace=False).tolist())]
    _compare(case, res, samp, DEFAULT, "max")
    out = gpu_run(case, scores_in=res["scores"], compact=False)
    check_selection_exact(case, out, units=units, rows_units=[])
