"""Per-layer budgets (tri_select_compact_layers) against the oracle.

The kept indices of every unit must equal the oracle's top-B of the GPU's
own scores with that unit's (sequence, layer) budget, found at the output
rows the oracle's out_rows_layers gives; compacted K, V and positions are
byte-exact gathers of the input rows.  Pyramid budgets come from the
library and must equal the oracle's pyramid_budgets.
"""
import numpy as np
import pytest
import torch

import oracle as O
import rope_aware_key_amd as R
import synth
from harness import gpu_run, pinned, shape_of, units_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _score(case):
    res = gpu_run(case, raw=False, stats=False, compact=False)
    return res["scores"]


def _run_layers(case, scores, budgets, with_rows=True):
    sh = shape_of(case)
    L, H, d = case.shape.num_layers, case.shape.num_kv_heads, case.shape.head_dim
    cu = pinned(case.cu_len, np.int64)
    bu = pinned(np.asarray(budgets, np.int32).reshape(-1), np.int32)
    lens = np.diff(case.cu_len)
    out_rows = int(sum(H * min(max(int(budgets[s][l]), 0), int(lens[s]))
                       for s in range(case.num_seqs) for l in range(L)))
    n_alloc = max(out_rows, 1)
    wsb = R.tri_workspace_bytes_layers(sh, cu)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV)
    kept = torch.full((n_alloc,), -1, dtype=torch.int32, device=DEV)
    k_out = v_out = pos_out = None
    if with_rows:
        k_out = torch.zeros((n_alloc, d), dtype=torch.int16, device=DEV)
        v_out = torch.zeros((n_alloc, d), dtype=torch.int16, device=DEV) if case.v is not None else None
        pos_out = torch.full((n_alloc,), -1, dtype=torch.int32, device=DEV)
    R.tri_select_compact_layers(sh, cu, bu, scores, case.k if with_rows else None,
                                case.v if with_rows else None, case.k_pos if with_rows else None,
                                kept, k_out, v_out, pos_out, workspace=ws)
    torch.cuda.synchronize()
    return out_rows, kept, k_out, v_out, pos_out


def _check(case, scores, budgets, out, units=None, rows_units=None):
    out_rows, kept, k_out, v_out, pos_out = out
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    sc = scores.cpu().numpy()
    kp = kept.cpu().numpy()
    units = units_of(case) if units is None else units
    rows_units = units if rows_units is None else rows_units
    covered = 0
    for (s, l, g) in units:
        start, n = case.unit_rows(s, l, g)
        ostart, b = O.out_rows_layers(case.cu_len, budgets, L, H, s, l, g)
        ref = O.select_topb(sc[start:start + n], int(budgets[s][l]))
        assert len(ref) == b
        np.testing.assert_array_equal(kp[ostart:ostart + b], ref, err_msg=f"unit {(s, l, g)}")
        covered += b
    for (s, l, g) in rows_units:
        start, n = case.unit_rows(s, l, g)
        ostart, b = O.out_rows_layers(case.cu_len, budgets, L, H, s, l, g)
        ref = O.select_topb(sc[start:start + n], int(budgets[s][l]))
        for name, src_t, out_t in (("k_out", case.k, k_out), ("v_out", case.v, v_out),
                                   ("pos_out", case.k_pos, pos_out)):
            if out_t is None or src_t is None:
                continue
            src = src_t[start:start + n].cpu().numpy()
            got = out_t[ostart:ostart + b].cpu().numpy()
            assert np.array_equal(got, O.compact_rows(src, ref)), f"{name} rows of unit {(s, l, g)}"
    if units is units_of(case) or len(units) == len(units_of(case)):
        assert covered == out_rows


def test_pyramid_budgets_library_equals_oracle():
    for L, mean, ratio in [(28, 2048, 3.0), (32, 1024, 2.0), (5, 100, 0.25), (1, 9.5, 3.0)]:
        np.testing.assert_array_equal(R.tri_pyramid_budgets(L, mean, ratio),
                                      O.pyramid_budgets(L, mean, ratio))


@pytest.mark.parametrize("seed", [0, 1])
def test_ragged_pyramid_budgets(seed):
    """Ragged batch with an empty sequence; per-sequence pyramids whose
    budgets fall below, at and above n, and a layer with budget 0."""
    shape = synth.Shape(128, 4, 2, 5)
    lens = [300, 0, 77, 1000]
    case = synth.build_case("layers_ragged", shape, lens, [1] * len(lens), device=DEV, seed=seed)
    budgets = np.stack([R.tri_pyramid_budgets(5, 150, 3.0),
                        R.tri_pyramid_budgets(5, 10, 2.0),
                        R.tri_pyramid_budgets(5, 77, 1.0),
                        R.tri_pyramid_budgets(5, 640, 4.0)]).astype(np.int32)
    budgets[3, 2] = 0
    budgets[2, 4] = 500
    scores = _score(case)
    _check(case, scores, budgets, _run_layers(case, scores, budgets))


def test_uniform_layers_equal_tri_select_compact():
    """One budget for every layer reproduces tri_select_compact exactly."""
    case = synth.workload_case("ragged", device=DEV, S=6, L=3, n_range=(100, 2500))
    res = gpu_run(case, raw=False, stats=False)
    budgets = np.repeat(case.budget[:, None], 3, axis=1).astype(np.int32)
    out = _run_layers(case, res["scores"], budgets)
    n = case.total_out_rows()
    assert out[0] == n
    for a, b in ((out[1], res["kept"]), (out[2], res["k_out"]), (out[3], res["v_out"]),
                 (out[4], res["pos_out"])):
        assert torch.equal(a[:n], b[:n])


def test_scores_only_selection():
    """K/V/positions absent: only kept indices are written."""
    shape = synth.Shape(64, 8, 2, 3)
    case = synth.build_case("layers_noval", shape, [513, 2049], [1, 1], device=DEV, seed=3,
                            with_values=False)
    budgets = np.array([[64, 128, 256], [1, 2048, 2049]], np.int32)
    scores = _score(case)
    _check(case, scores, budgets, _run_layers(case, scores, budgets, with_rows=False))


def test_long_units_split_select():
    """Units past 35840 keys (split select over 4096-key tiles) with
    per-layer budgets: a short sequence in the same batch, budgets of 0, 1,
    n - 1 and above n, ties on a few score values across every tile."""
    shape = synth.Shape(64, 4, 2, 3)
    lens = [41000, 900, 70000]
    case = synth.build_case("layers_long", shape, lens, [1] * len(lens), device=DEV, seed=9)
    g = np.random.default_rng(9)
    sc = (g.integers(-4, 5, size=case.total_rows()) * 0.25).astype(np.float32)
    scores = torch.as_tensor(sc, device=DEV)
    budgets = np.array([[0, 40999, 50000], [1, 899, 4096], [1, 69999, 12345]], np.int32)
    _check(case, scores, budgets, _run_layers(case, scores, budgets),
           rows_units=[(0, 1, 0), (2, 2, 1), (1, 1, 1)])


def test_long_reasoning_pyramid_full_size():
    """8 x 32768 keys, 28 layers, pyramid mean 2048 ratio 3: every unit's
    kept set checked; rows checked on sampled units."""
    case = synth.workload_case("long_reasoning", device=DEV)
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    pyr = R.tri_pyramid_budgets(L, 2048, 3.0)
    budgets = np.repeat(pyr[None, :], case.num_seqs, axis=0).astype(np.int32)
    scores = _score(case)
    out = _run_layers(case, scores, budgets)
    assert out[0] == case.num_seqs * H * int(pyr.sum())
    rng = np.random.default_rng(5)
    units = units_of(case)
    sample = [units[i] for i in sorted(rng.choice(len(units), 12, replace=False))]
    sample += [(0, 0, 0), (case.num_seqs - 1, L - 1, H - 1)]
    _check(case, scores, budgets, out, units=units, rows_units=sample)
