"""Seeded random sweep of the whole path against the oracle.

Each case draws a head_dim (any multiple of 8 up to 256), a GQA group (1 to
16), a small ragged batch, the RoPE layout, the offset set and its
reduction, and whether K sits in a paged pool (page size and order drawn
too).  Bars as elsewhere: scores within 1e-4 * max(1, |ref|) (floored at
the fp32 resolution of the raw scores), raw scores and per-head statistics
against the oracle, selection bit-exact on the GPU's own scores, compacted
rows byte-exact.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import (check_raw, check_scores, check_selection_exact, gpu_run, gpu_score_offsets,
                     gpu_score_paged, half_split, oracle_unit, units_of, z_floor)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def draw(seed):
    g = np.random.default_rng([91, seed])
    # half the cases on the MFMA kernels' head dims (multiples of 32)
    d = int(g.integers(1, 9)) * 32 if g.random() < 0.5 else int(g.integers(1, 33)) * 8
    G = int(g.integers(1, 17))
    Hkv = int(g.integers(1, 4))
    L = int(g.integers(1, 3))
    S = int(g.integers(1, 5))
    lens = [int(x) for x in g.integers(0, 2500, size=S)]
    budgets = [int(x) for x in g.integers(0, 2600, size=S)]
    half = bool(g.integers(0, 2))
    reduce = "max" if (d % 32 == 0 and (not half or d % 64 == 0) and g.random() < 0.4) else "mean"
    offsets = None
    if reduce == "max" or g.random() < 0.3:
        n_off = int(g.integers(1, 18))
        offsets = sorted(float(x) for x in g.choice(70000, size=n_off, replace=False))
    paged = bool(g.integers(0, 2))
    page = int(2 ** g.integers(0, 9)) if paged else None
    head_major = bool(g.integers(0, 2))
    return dict(d=d, G=G, Hkv=Hkv, L=L, lens=lens, budgets=budgets, half=half, reduce=reduce,
                offsets=offsets, page=page, head_major=head_major)


@pytest.mark.parametrize("seed", range(512))
def test_random_case(seed):
    c = draw(seed)
    print(f"random case {seed}: {c}", flush=True)
    shape = synth.Shape(c["d"], c["G"] * c["Hkv"], c["Hkv"], c["L"])
    case = synth.build_case("random", shape, c["lens"], c["budgets"], device=DEV, seed=seed)
    if c["half"]:
        case = half_split(case)
    if c["page"] is not None:
        pool = synth.paged_from_case(case, c["page"], head_major=c["head_major"], seed=seed)
        res = gpu_score_paged(case, pool, c["offsets"], c["reduce"], raw=True, stats=True)
    elif c["offsets"] is not None:
        res = gpu_score_offsets(case, c["offsets"], c["reduce"], raw=True, stats=True)
    else:
        res = gpu_run(case, raw=True, stats=True, compact=False)
    scores = res["scores"].cpu().numpy()
    raw = res["raw"].cpu().numpy()
    hs = res["head_stats"].cpu().numpy()
    L, H = c["L"], c["Hkv"]
    for (s, l, g) in units_of(case):
        if case.seq_len(s) == 0:
            continue
        start, n, ref, S, mu, sigma = oracle_unit(case, s, l, g, factored=True,
                                                  offsets=c["offsets"], reduce=c["reduce"])
        what = f"case {seed} unit {(s, l, g)}"
        check_scores(scores[start:start + n], ref, what, z_floor(S, sigma))
        check_raw(raw[start:start + n], S, sigma, "raw " + what)
        u = (s * L + l) * H + g
        top = max(np.max(sigma), np.max(np.abs(S)))
        np.testing.assert_allclose(hs[u, :, 0], mu, rtol=0, atol=1e-5 * top, err_msg=what)
        np.testing.assert_allclose(hs[u, :, 1], sigma, rtol=1e-5, atol=1e-5 * np.max(np.abs(S)),
                                   err_msg=what)
    sel = gpu_run(case, scores_in=res["scores"])
    check_selection_exact(case, sel)


@pytest.mark.parametrize("seed", range(24))
def test_random_select_variants(seed):
    """Per-layer budgets (tri_select_compact_layers) and paged compaction
    (tri_select_compact_paged, another page size and order for the output)
    on random batches, against the oracle's selection on the GPU's scores."""
    import rope_aware_key_amd as R
    from harness import pinned, shape_of
    g = np.random.default_rng([95, seed])
    d = int(g.integers(1, 33)) * 8
    G, Hkv, L = int(g.integers(1, 9)), int(g.integers(1, 4)), int(g.integers(1, 4))
    S = int(g.integers(1, 5))
    lens = [int(x) for x in g.integers(0, 3000, size=S)]
    budgets = [int(x) for x in g.integers(0, 3100, size=S)]
    shape = synth.Shape(d, G * Hkv, Hkv, L)
    case = synth.build_case("random_sel", shape, lens, budgets, device=DEV, seed=seed)
    scores = gpu_run(case, raw=False, stats=False, compact=False)["scores"]
    sc = scores.cpu().numpy()
    sh = shape_of(case)
    cu = pinned(case.cu_len, np.int64)
    # per-layer budgets
    lb = g.integers(0, 3100, size=(S, L)).astype(np.int32)
    out_rows = int(sum(Hkv * min(int(lb[s, l]), case.seq_len(s)) for s in range(S) for l in range(L)))
    kept = torch.full((max(out_rows, 1),), -1, dtype=torch.int32, device=DEV)
    ko = torch.zeros((max(out_rows, 1), d), dtype=torch.int16, device=DEV)
    ws = torch.empty(max(R.tri_workspace_bytes_layers(sh, cu), 1), dtype=torch.uint8, device=DEV)
    R.tri_select_compact_layers(sh, cu, pinned(lb.reshape(-1), np.int32), scores, case.k, None,
                                None, kept, ko, None, None, workspace=ws)
    torch.cuda.synchronize()
    kp, kop, kin = kept.cpu().numpy(), ko.cpu().numpy(), case.k.cpu().numpy()
    for (s, l, gg) in units_of(case):
        start, n = case.unit_rows(s, l, gg)
        ostart, b = O.out_rows_layers(case.cu_len, lb, L, Hkv, s, l, gg)
        ref = O.select_topb(sc[start:start + n], int(lb[s, l]))
        np.testing.assert_array_equal(kp[ostart:ostart + b], ref, err_msg=f"layers {(s, l, gg)}")
        assert np.array_equal(kop[ostart:ostart + b], kin[start:start + n][ref])
    # paged in, paged out
    P_in, P_out = int(2 ** g.integers(0, 9)), int(2 ** g.integers(0, 9))
    pool = synth.paged_from_case(case, P_in, head_major=bool(g.integers(0, 2)), seed=seed)
    need = [(case.kept(s) + P_out - 1) // P_out for s in range(S)]
    out = synth.empty_pool(S, L, Hkv, d, P_out, need, bool(g.integers(0, 2)), spare=1,
                           seed=seed + 1, device=DEV)
    kept2 = torch.full((max(case.total_out_rows(), 1),), -1, dtype=torch.int32, device=DEV)
    ws2 = torch.empty(max(R.tri_workspace_bytes(sh, cu), 1), dtype=torch.uint8, device=DEV)
    pin = R.make_pages(pool.table, P_in, pool.num_pages, *pool.strides())
    pout = R.make_pages(out.table, P_out, out.num_pages, *out.strides())
    R.tri_select_compact_paged(sh, cu, pinned(case.budget, np.int32), scores, pin, pool.k, pool.v,
                               pool.pos, kept2, pout, out.k, out.v, out.pos, workspace=ws2)
    torch.cuda.synchronize()
    k2 = kept2.cpu().numpy()
    for (s, l, gg) in units_of(case):
        start, n = case.unit_rows(s, l, gg)
        ostart, b = case.unit_out_rows(s, l, gg)
        ref = O.select_topb(sc[start:start + n], int(case.budget[s]))
        np.testing.assert_array_equal(k2[ostart:ostart + b], ref, err_msg=f"paged {(s, l, gg)}")
        if b:
            rows = torch.as_tensor(out.unit_rows(s, l, gg, b), device=DEV)
            src = case.k[start:start + n].cpu().numpy()[ref]
            assert np.array_equal(out.k[rows].cpu().numpy(), src), f"paged K {(s, l, gg)}"
            srcp = case.k_pos[start:start + n].cpu().numpy()[ref]
            assert np.array_equal(out.pos[rows].cpu().numpy(), srcp), f"paged pos {(s, l, gg)}"


@pytest.mark.parametrize("seed", range(12))
def test_random_select_long_units(seed):
    """Batches whose longest unit has 4096 < n <= 32768 keys, so selection
    and gathers run fused in one kernel per unit (register-held keys), at
    any head_dim (multiple of 8: 1 to 32 lanes per row), with per-layer
    budgets and paged pools too.  Scores are drawn directly (normals with a
    share of repeated values, NaN and signed zeros), and selection and
    gathered rows are compared exactly with the oracle's selection."""
    import rope_aware_key_amd as R
    from harness import pinned, shape_of
    g = np.random.default_rng([97, seed])
    d = int(g.integers(1, 33)) * 8
    G, Hkv, L = int(g.integers(1, 5)), int(g.integers(1, 3)), int(g.integers(1, 3))
    S = int(g.integers(1, 4))
    lens = [int(x) for x in g.integers(0, 32769, size=S)]
    lens[int(g.integers(0, S))] = int(g.integers(4097, 32769))
    budgets = [int(x) for x in g.integers(0, 33000, size=S)]
    shape = synth.Shape(d, G * Hkv, Hkv, L)
    case = synth.build_case("random_long", shape, lens, budgets, device=DEV, seed=seed)
    rows = case.total_rows()
    sc = g.normal(size=rows).astype(np.float32)
    ties = g.random(rows) < 0.2
    sc[ties] = np.round(sc[ties] * 2) / 2
    sc[g.random(rows) < 0.01] = np.nan
    sc[g.random(rows) < 0.01] = -0.0
    scores = torch.as_tensor(sc, device=DEV)
    # packed
    res = gpu_run(case, scores_in=scores)
    check_selection_exact(case, res)
    sh = shape_of(case)
    cu = pinned(case.cu_len, np.int64)
    # per-layer budgets
    lb = g.integers(0, 33000, size=(S, L)).astype(np.int32)
    out_rows = int(sum(Hkv * min(int(lb[s, l]), case.seq_len(s)) for s in range(S) for l in range(L)))
    kept = torch.full((max(out_rows, 1),), -1, dtype=torch.int32, device=DEV)
    ko = torch.zeros((max(out_rows, 1), d), dtype=torch.int16, device=DEV)
    ws = torch.empty(max(R.tri_workspace_bytes_layers(sh, cu), 1), dtype=torch.uint8, device=DEV)
    R.tri_select_compact_layers(sh, cu, pinned(lb.reshape(-1), np.int32), scores, case.k, None,
                                None, kept, ko, None, None, workspace=ws)
    torch.cuda.synchronize()
    kp, kop, kin = kept.cpu().numpy(), ko.cpu().numpy(), case.k.cpu().numpy()
    for (s, l, gg) in units_of(case):
        start, n = case.unit_rows(s, l, gg)
        ostart, b = O.out_rows_layers(case.cu_len, lb, L, Hkv, s, l, gg)
        ref = O.select_topb(sc[start:start + n], int(lb[s, l]))
        np.testing.assert_array_equal(kp[ostart:ostart + b], ref, err_msg=f"layers {(s, l, gg)}")
        assert np.array_equal(kop[ostart:ostart + b], kin[start:start + n][ref])
    # paged in, paged out
    P_in, P_out = int(2 ** g.integers(0, 9)), int(2 ** g.integers(0, 9))
    pool = synth.paged_from_case(case, P_in, head_major=bool(g.integers(0, 2)), seed=seed)
    need = [(case.kept(s) + P_out - 1) // P_out for s in range(S)]
    out = synth.empty_pool(S, L, Hkv, d, P_out, need, bool(g.integers(0, 2)), spare=1,
                           seed=seed + 1, device=DEV)
    kept2 = torch.full((max(case.total_out_rows(), 1),), -1, dtype=torch.int32, device=DEV)
    ws2 = torch.empty(max(R.tri_workspace_bytes(sh, cu), 1), dtype=torch.uint8, device=DEV)
    pin = R.make_pages(pool.table, P_in, pool.num_pages, *pool.strides())
    pout = R.make_pages(out.table, P_out, out.num_pages, *out.strides())
    R.tri_select_compact_paged(sh, cu, pinned(case.budget, np.int32), scores, pin, pool.k, pool.v,
                               pool.pos, kept2, pout, out.k, out.v, out.pos, workspace=ws2)
    torch.cuda.synchronize()
    k2 = kept2.cpu().numpy()
    for (s, l, gg) in units_of(case):
        start, n = case.unit_rows(s, l, gg)
        ostart, b = case.unit_out_rows(s, l, gg)
        ref = O.select_topb(sc[start:start + n], int(case.budget[s]))
        np.testing.assert_array_equal(k2[ostart:ostart + b], ref, err_msg=f"paged {(s, l, gg)}")
        if b:
            rows_ = torch.as_tensor(out.unit_rows(s, l, gg, b), device=DEV)
            src = case.k[start:start + n].cpu().numpy()[ref]
            assert np.array_equal(out.k[rows_].cpu().numpy(), src), f"paged K {(s, l, gg)}"
            srcv = case.v[start:start + n].cpu().numpy()[ref]
            assert np.array_equal(out.v[rows_].cpu().numpy(), srcv), f"paged V {(s, l, gg)}"
            srcp = case.k_pos[start:start + n].cpu().numpy()[ref]
            assert np.array_equal(out.pos[rows_].cpu().numpy(), srcp), f"paged pos {(s, l, gg)}"
