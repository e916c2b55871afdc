"""The process-pool comparison the full-size parity tests use, on the CPU:
results taken from the oracle itself pass with zero error on every unit,
and one planted score error, or one wrong sigma, fails naming its unit."""
import numpy as np
import pytest
import torch

import synth
from harness import compare_units_pool, oracle_unit, units_of


def _oracle_results(case):
    G = case.shape.group
    scores = torch.zeros(case.total_rows(), dtype=torch.float32)
    hs = torch.zeros(case.num_units, G, 2, dtype=torch.float64)
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    for (s, l, g) in units_of(case):
        if case.seq_len(s) == 0:
            continue
        start, n, ref, S, mu, sigma = oracle_unit(case, s, l, g, factored=True)
        scores[start:start + n] = torch.as_tensor(ref, dtype=torch.float32)
        u = (s * L + l) * H + g
        hs[u, :, 0] = torch.as_tensor(mu)
        hs[u, :, 1] = torch.as_tensor(sigma)
    return {"scores": scores, "head_stats": hs}


@pytest.fixture(scope="module")
def case():
    return synth.build_case("pool", synth.Shape(64, 8, 2, 2), [300, 0, 517], [64, 8, 100], seed=9)


def test_pool_passes_oracle_results(case):
    res = _oracle_results(case)
    worst, floors = compare_units_pool(case, res, units_of(case))
    assert worst <= 1e-6 and len(floors) == len(units_of(case))


def test_pool_names_a_planted_score_error(case):
    res = _oracle_results(case)
    units = units_of(case)
    s, l, g = units[-1]
    start, n = case.unit_rows(s, l, g)
    res["scores"][start + n // 2] += 1e-3
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    with pytest.raises(AssertionError, match=f"unit {(s * L + l) * H + g}:"):
        compare_units_pool(case, res, units)


def test_pool_names_a_wrong_sigma(case):
    res = _oracle_results(case)
    res["head_stats"][1, 3, 1] *= 1.001
    with pytest.raises(AssertionError, match="unit 1: head stats"):
        compare_units_pool(case, res, units_of(case))
