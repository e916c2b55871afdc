"""Paged K/V/position pools (tri_score_paged, tri_select_compact_paged).

Each case is a packed synthetic case scattered into a pool with random page
order and garbage in the spare pages.  Where the paged call runs the same
kernel as the packed call (pages of >= 16 tokens, or the VALU path on
both), its scores must equal the packed scores bit for bit; otherwise
they are held to the oracle (|gpu - ref| <= 1e-4 * max(1, |ref|)).
Kept indices must equal the packed call's, and every compacted row in the
output pool must equal the packed compaction's row byte for byte.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import (check_scores, check_selection_exact, gpu_run, gpu_score_offsets,
                     gpu_score_paged, half_split, oracle_unit, pinned, shape_of, units_of)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _paged_score(case, pool, offsets=None, reduce="mean", raw=False, stats=False):
    return gpu_score_paged(case, pool, offsets, reduce, raw, stats)


def _paged_select(case, scores, pool, out_page_size, head_major_out=False):
    import rope_aware_key_amd as R
    sh = shape_of(case)
    S, L, H, d = case.num_seqs, case.shape.num_layers, case.shape.num_kv_heads, case.shape.head_dim
    cu = pinned(case.cu_len, np.int64)
    bu = pinned(case.budget, np.int32)
    need = [(case.kept(s) + out_page_size - 1) // out_page_size for s in range(S)]
    out = synth.empty_pool(S, L, H, d, out_page_size, need, head_major_out, spare=2, seed=5,
                           device=DEV, with_values=case.v is not None)
    ws = torch.empty(max(R.tri_workspace_bytes(sh, cu), 1), dtype=torch.uint8, device=DEV)
    kept = torch.full((max(case.total_out_rows(), 1),), -1, dtype=torch.int32, device=DEV)
    pin = R.make_pages(pool.table, pool.page_size, pool.num_pages, *pool.strides())
    pout = R.make_pages(out.table, out.page_size, out.num_pages, *out.strides())
    R.tri_select_compact_paged(sh, cu, bu, scores, pin, pool.k, pool.v, pool.pos, kept, pout, out.k,
                               out.v, out.pos, workspace=ws)
    torch.cuda.synchronize()
    return kept[:case.total_out_rows()], out


def _check_rows(case, res, out, units):
    """Output pool rows of every unit equal the packed compaction's rows."""
    for (s, l, g) in units:
        ostart, b = case.unit_out_rows(s, l, g)
        if b == 0:
            continue
        rows = torch.as_tensor(out.unit_rows(s, l, g, b), device=DEV)
        assert torch.equal(out.k[rows], res["k_out"][ostart:ostart + b]), f"K of {(s, l, g)}"
        if case.v is not None:
            assert torch.equal(out.v[rows], res["v_out"][ostart:ostart + b]), f"V of {(s, l, g)}"
        assert torch.equal(out.pos[rows], res["pos_out"][ostart:ostart + b]), f"pos of {(s, l, g)}"


def _bits(t):
    return t.view(torch.int32)


def test_pool_rows_follow_the_oracle():
    case = synth.build_case("pool", synth.Shape(64, 4, 2, 2), [37, 0, 100], [5, 5, 5], seed=1)
    for hm in (False, True):
        pool = synth.paged_from_case(case, 16, head_major=hm)
        tab = pool.table.cpu().numpy()
        for (s, l, g) in units_of(case):
            n = case.seq_len(s)
            np.testing.assert_array_equal(pool.unit_rows(s, l, g, n),
                                          O.paged_unit_rows(tab, 16, pool.strides(), s, l, g, n))


@pytest.mark.parametrize("d,G,P,head_major,P_out", [
    (128, 4, 16, False, 16), (128, 7, 64, True, 32), (64, 2, 256, False, 8), (256, 2, 32, True, 64)])
def test_paged_equals_packed_bitwise(d, G, P, head_major, P_out):
    """Fused MFMA path (pages >= 16 tokens): scores, raw scores and
    statistics bit-identical to the packed call; selection and compacted
    rows identical."""
    shape = synth.Shape(d, 2 * G, 2, 2)
    case = synth.build_case("paged", shape, [300, 0, 1000, 2100, 17], [128, 5, 1000, 3000, 9],
                            device=DEV, seed=d + P)
    res = gpu_run(case, raw=True, stats=True)
    pool = synth.paged_from_case(case, P, head_major=head_major, seed=P)
    pr = _paged_score(case, pool, raw=True, stats=True)
    assert torch.equal(_bits(pr["scores"]), _bits(res["scores"]))
    assert torch.equal(pr["raw"].view(torch.int32), res["raw"].view(torch.int32))
    assert torch.equal(pr["head_stats"].view(torch.int64), res["head_stats"].view(torch.int64))
    kept, out = _paged_select(case, res["scores"], pool, P_out)
    assert torch.equal(kept, res["kept"])
    _check_rows(case, res, out, units_of(case))


def test_paged_long_units_split_select():
    """Units past 35840 keys in a paged pool: the split select on the scores
    and the compaction through both page tables give the packed call's kept
    indices and rows; a short sequence shares the batch."""
    shape = synth.Shape(64, 8, 2, 1)
    case = synth.build_case("paged_long", shape, [40000, 700, 65536], [20000, 699, 4096],
                            device=DEV, seed=23)
    res = gpu_run(case, raw=False, stats=False)
    pool = synth.paged_from_case(case, 64, head_major=True, seed=23)
    pr = _paged_score(case, pool)
    assert torch.equal(_bits(pr["scores"]), _bits(res["scores"]))
    kept, out = _paged_select(case, res["scores"], pool, 128)
    assert torch.equal(kept, res["kept"])
    _check_rows(case, res, out, units_of(case))
    check_selection_exact(case, res, rows_units=[])


@pytest.mark.parametrize("P", [1, 4, 8])
def test_small_pages_valu_path(P):
    """Pages under 16 tokens take the VALU path: scores against the oracle;
    selection and rows against the packed call on the same scores."""
    shape = synth.Shape(128, 8, 2, 1)
    case = synth.build_case("paged_small", shape, [129, 40, 0, 333], [64, 100, 3, 100],
                            device=DEV, seed=P)
    pool = synth.paged_from_case(case, P, seed=P)
    pr = _paged_score(case, pool)
    sc = pr["scores"].cpu().numpy()
    for (s, l, g) in units_of(case):
        if case.seq_len(s) == 0:
            continue
        start, n, ref, _, _, _ = oracle_unit(case, s, l, g, factored=True)
        check_scores(sc[start:start + n], ref, f"paged P={P} unit {(s, l, g)}")
    res = gpu_run(case, raw=False, stats=False, scores_in=pr["scores"])
    kept, out = _paged_select(case, pr["scores"], pool, 4, head_major_out=True)
    assert torch.equal(kept, res["kept"])
    _check_rows(case, res, out, units_of(case))


def test_paged_valu_head_dim_bitwise():
    """head_dim 48 takes the VALU path both ways: bit-identical scores."""
    shape = synth.Shape(48, 6, 2, 2)
    case = synth.build_case("paged48", shape, [77, 500], [10, 100], device=DEV, seed=3)
    res = gpu_run(case, raw=False, stats=True)
    pr = _paged_score(case, synth.paged_from_case(case, 32, head_major=True), stats=True)
    assert torch.equal(_bits(pr["scores"]), _bits(res["scores"]))
    assert torch.equal(pr["head_stats"].view(torch.int64), res["head_stats"].view(torch.int64))


@pytest.mark.parametrize("reduce", ["mean", "max"])
def test_paged_offsets_bitwise(reduce):
    offs = [float(x) for x in range(1, 129, 8)]
    shape = synth.Shape(128, 8, 2, 1)
    case = synth.build_case("paged_off", shape, [700, 64, 2049], [1, 1, 1], device=DEV, seed=11)
    res = gpu_score_offsets(case, offs, reduce, raw=False, stats=True)
    pr = _paged_score(case, synth.paged_from_case(case, 16), offsets=offs, reduce=reduce,
                      stats=True)
    assert torch.equal(_bits(pr["scores"]), _bits(res["scores"]))
    assert torch.equal(pr["head_stats"].view(torch.int64), res["head_stats"].view(torch.int64))


def test_paged_half_split_bitwise():
    shape = synth.Shape(128, 8, 2, 2)
    case = half_split(synth.build_case("paged_half", shape, [1000, 31], [100, 4], device=DEV,
                                       seed=12))
    res = gpu_run(case, raw=False, stats=False, compact=False)
    pr = _paged_score(case, synth.paged_from_case(case, 64, head_major=True))
    assert torch.equal(_bits(pr["scores"]), _bits(res["scores"]))


def test_out_of_range_page_ids_are_clamped():
    """Ids outside [0, num_pages) read a page inside the pool (no access
    outside it); the call completes and every score is finite."""
    shape = synth.Shape(128, 4, 2, 1)
    case = synth.build_case("clamp", shape, [100, 60], [10, 10], device=DEV, seed=13)
    pool = synth.paged_from_case(case, 16)
    pool.table[0, 1] = -7
    pool.table[1, 0] = pool.num_pages + 5
    pr = _paged_score(case, pool)
    assert torch.isfinite(pr["scores"]).all()
    pool2 = synth.paged_from_case(case, 4)
    pool2.table[0, 3] = -1
    pool2.table[1, 2] = 1 << 30
    pr2 = _paged_score(case, pool2)
    assert torch.isfinite(pr2["scores"]).all()


@pytest.mark.timeout(600)
def test_long_reasoning_paged_full_size():
    """The 32K -> 2048 workload in 16-token token-major pages: scores equal
    the packed call's on every unit; selection equal; rows of sampled units
    equal in a 64-token output pool."""
    case = synth.workload_case("long_reasoning", device=DEV)
    res = gpu_run(case, raw=False, stats=False)
    pool = synth.paged_from_case(case, 16, seed=21)
    pr = _paged_score(case, pool)
    assert torch.equal(_bits(pr["scores"]), _bits(res["scores"]))
    kept, out = _paged_select(case, res["scores"], pool, 64)
    assert torch.equal(kept, res["kept"])
    g = np.random.default_rng(4)
    units = units_of(case)
    _check_rows(case, res, out, [units[i] for i in g.choice(len(units), 6, replace=False)])
