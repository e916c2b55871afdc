"""Parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (scores are z-scores, in units of the per-head sigma):
  scores      |gpu - ref| <= 1e-4 * max(1, |ref|)
  raw S~_h    |gpu - ref| <= 1e-4 * max(|ref|, sigma_h)
  statistics  relative 1e-5 (calibration), mu/sigma relative 1e-5 of sigma
  selection   bit-exact against the oracle's selection on the GPU's own scores
  compaction  byte-exact
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import (z_floor, check_kept_near_threshold, check_raw, check_scores, check_selection_exact,
                     compare_units_pool, gpu_calibrate, gpu_run, oracle_unit, units_of)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _compare_units(case, res, units, factored, floors=False):
    """Units against the oracle one by one; returns the worst score error
    (and, with floors=True, every unit's z_floor)."""
    scores = res["scores"].cpu().numpy()
    raw = res["raw"].cpu().numpy() if res.get("raw") is not None else None
    hs = res["head_stats"].cpu().numpy() if res.get("head_stats") is not None else None
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    worst, fl = 0.0, []
    for (s, l, g) in units:
        if case.seq_len(s) == 0:
            continue
        start, n, ref, S, mu, sigma = oracle_unit(case, s, l, g, factored=factored)
        fl.append(z_floor(S, sigma))
        worst = max(worst, check_scores(scores[start:start + n], ref, f"unit {(s, l, g)}", fl[-1]))
        if raw is not None:
            check_raw(raw[start:start + n], S, sigma, f"raw unit {(s, l, g)}")
        if hs is not None:
            u = (s * L + l) * H + g
            np.testing.assert_allclose(hs[u, :, 0], mu, rtol=0, atol=1e-5 * max(np.max(sigma), np.max(np.abs(S))))
            np.testing.assert_allclose(hs[u, :, 1], sigma, rtol=1e-5, atol=1e-5 * np.max(np.abs(S)))
    return (worst, fl) if floors else worst


# ------------------------------------------------------------- calibration
def test_calibrate_smallest_matches_oracle():
    case = synth.workload_case("smallest", device=DEV)
    gpu_calibrate(case)
    q = O.bf16_bits_to_f64(case.calib_q[0].cpu().numpy().view(np.uint16))   # [N, Hq, d]
    om = O.rope_omega(128, 1e4)
    centre, absmean, Rr = O.calibrate(q, case.calib_pos.cpu().numpy(), om)
    qc = case.q_centre[0].cpu().double().numpy()
    np.testing.assert_allclose(qc[..., 0], centre.real, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(qc[..., 1], centre.imag, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(case.q_absmean[0].cpu().double().numpy(), absmean, rtol=1e-5)
    np.testing.assert_allclose(case.q_R[0].cpu().double().numpy(), Rr, rtol=1e-5)
    assert 0.9 < float(Rr.mean()) < 0.99     # the synthetic queries are concentrated


def test_calibrate_pre_rope_and_multi_layer():
    torch.manual_seed(0)
    L, N, Hq, d = 2, 257, 3, 16
    q = (torch.randn(L, N, Hq, d, device=DEV) + 0.7).to(torch.bfloat16).view(torch.int16)
    import rope_aware_key_amd as R
    sh = R.make_shape(d, Hq, 1, L)
    c = torch.empty(L, Hq, d // 2, 2, device=DEV)
    a = torch.empty(L, Hq, d // 2, device=DEV)
    r = torch.empty(L, Hq, d // 2, device=DEV)
    R.tri_calibrate(sh, q, None, N, c, a, r)
    torch.cuda.synchronize()
    qq = O.bf16_bits_to_f64(q.cpu().numpy().view(np.uint16))
    om = O.rope_omega(d, 1e4)
    for l in range(L):
        centre, absmean, Rr = O.calibrate(qq[l], None, om)
        np.testing.assert_allclose(c[l, ..., 0].cpu().numpy(), centre.real, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(c[l, ..., 1].cpu().numpy(), centre.imag, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(a[l].cpu().numpy(), absmean, rtol=1e-5)
        np.testing.assert_allclose(r[l].cpu().numpy(), Rr, rtol=1e-5)


# ------------------------------------------------------ smallest, end to end
def test_smallest_end_to_end_term_by_term():
    """Smallest workload in full: GPU calibration -> score -> select/compact,
    against the oracle's own calibration and term-by-term scores."""
    case = synth.workload_case("smallest", device=DEV)
    gpu_calibrate(case)
    res = gpu_run(case)
    q = O.bf16_bits_to_f64(case.calib_q[0].cpu().numpy().view(np.uint16))
    om = O.rope_omega(128, 1e4)
    stats = O.calibrate(q, case.calib_pos.cpu().numpy(), om)
    start, n, ref, S, mu, sigma = oracle_unit(case, 0, 0, 0, factored=False, stats=stats)
    assert z_floor(S, sigma) <= 1e-4      # the plain bar holds; no fp32-resolution floor
    check_scores(res["scores"].cpu().numpy(), ref, "smallest")
    check_raw(res["raw"].cpu().numpy(), S, sigma, "smallest raw")
    check_selection_exact(case, res)
    # end-to-end kept set vs the oracle's own selection on fp64 scores
    b = case.kept(0)
    ref_kept = set(O.select_topb(ref, b).tolist())
    got = set(res["kept"].cpu().numpy().tolist())
    thr = np.sort(ref)[::-1][b - 1]
    diff = ref_kept ^ got
    assert all(abs(ref[i] - thr) <= 1e-4 * max(1.0, abs(thr)) for i in diff), sorted(diff)[:10]


# ------------------------------------------- reduced configs, many tiles
REDUCED = {
    "decode_window": dict(S=2, L=1),                # 16 units, n = 3200 (3 tiles + tail)
    "long_reasoning": dict(S=1, L=1, n=5000, B=2048),  # G = 7, 4 tiles + ragged tail
    "ragged": dict(S=6, L=1, n_range=(100, 3000)),  # ragged lengths, some B >= n
    "stress_ties": dict(n=5000, B=1024),            # d = 64, G = 8, duplicated blocks
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_reduced_config_parity(name):
    case = synth.workload_case(name, device=DEV, **REDUCED[name])
    res = gpu_run(case)
    units = units_of(case)
    # every unit against the factored oracle path, two against term-by-term
    _compare_units(case, res, units, factored=True)
    _compare_units(case, res, units[:1] + units[-1:], factored=False)
    check_selection_exact(case, res)
    check_kept_near_threshold(case, res, units)


@pytest.mark.parametrize("d,G", [(48, 3), (96, 5), (256, 2), (32, 16)])
def test_other_head_dims(d, G):
    """head_dim 48 takes the generic VALU kernels; multiples of 32 take the
    fused MFMA kernel (one MFMA step at d = 32, eight at d = 256)."""
    shape = synth.Shape(d, 2 * G, 2, 2)
    case = synth.build_case("dims", shape, [1500, 2100, 0, 37], [300, 2100, 5, 40], device=DEV, seed=d)
    res = gpu_run(case)
    units = units_of(case)
    _compare_units(case, res, units, factored=True)
    check_selection_exact(case, res)
    check_kept_near_threshold(case, res, units)


def test_duplicate_keys_score_bitwise_equal():
    case = synth.workload_case("stress_ties", device=DEV, n=4096, B=512)
    res = gpu_run(case, raw=False, stats=False, compact=False)
    sc = res["scores"].cpu().numpy()
    for (s, l, g) in units_of(case):
        start, n = case.unit_rows(s, l, g)
        u = sc[start:start + n].reshape(-1, 128)
        assert np.array_equal(u[:, 64:].view(np.uint32), u[:, :64].view(np.uint32))
    check_selection_exact(case, res)


def test_determinism_bitwise():
    case = synth.workload_case("long_reasoning", device=DEV, S=1, L=2, n=3000, B=700)
    a = gpu_run(case)
    b = gpu_run(case)
    for key in ("scores", "raw", "head_stats", "kept", "k_out", "v_out", "pos_out"):
        assert torch.equal(a[key].view(torch.uint8) if a[key].dtype.is_floating_point else a[key],
                           b[key].view(torch.uint8) if b[key].dtype.is_floating_point else b[key]), key


# ----------------------------------------------- hand-built selection cases
def _hand_case(lens, budgets, d=64, L=1, Hkv=2, G=1):
    shape = synth.Shape(d, Hkv * G, Hkv, L)
    return synth.build_case("hand", shape, lens, budgets, device=DEV, seed=3)


def test_select_edge_cases_exact():
    lens = [0, 1, 5, 1025, 3000, 700, 2049]
    budgets = [4, 0, 9, 1025, 17, 3, 2048]
    case = _hand_case(lens, budgets)
    rows = case.total_rows()
    g = np.random.default_rng(7)
    pool = np.array([0.0, -0.0, 1.5, -1.5, np.inf, -np.inf, np.nan, 3.25, 1e-38, -1e-38], np.float32)
    sc = g.choice(pool, size=rows).astype(np.float32)
    # one unit with all-equal scores, one with random normals
    s0, n0 = case.unit_rows(4, 0, 1)
    sc[s0:s0 + n0] = 2.0
    s1, n1 = case.unit_rows(6, 0, 0)
    sc[s1:s1 + n1] = g.normal(size=n1).astype(np.float32)
    scores = torch.as_tensor(sc, device=DEV)
    res = gpu_run(case, scores_in=scores)
    check_selection_exact(case, res)
    ostart, b = case.unit_out_rows(4, 0, 1)
    np.testing.assert_array_equal(res["kept"][ostart:ostart + b].cpu().numpy(), np.arange(17))


@pytest.mark.parametrize("n,B", [(4096, 4095), (4096, 1), (20000, 10000), (33000, 2048),
                                 (4097, 4096), (35840, 1)])
def test_select_many_ties(n, B):
    case = _hand_case([n], [B], Hkv=1)
    g = np.random.default_rng(n + B)
    sc = g.integers(-3, 4, size=n).astype(np.float32) * 0.5    # 7 distinct values
    res = gpu_run(case, scores_in=torch.as_tensor(sc, device=DEV))
    check_selection_exact(case, res)


def test_select_held_edge_cases_exact():
    """A batch whose longest unit (32768 keys) takes the register-held
    select (16384 < n <= 32768: 32 keys per lane, places past n padded with
    the NaN key): empty, single-key, fully kept and budget-0 units, lengths
    that leave waves partly or wholly past n; NaN, signed zeros, infinities
    and denormals; an all-equal unit (the top-digit list overflows, so the
    lower digits come from the held keys); a unit whose threshold is the
    NaN key itself, so that the kept NaNs come first in index order and no
    padding place may be taken; and normal scores."""
    lens = [0, 1, 5, 64, 4097, 32768, 20000, 9999, 16385, 20001]
    budgets = [4, 0, 9, 64, 1, 32767, 2, 9998, 6000, 5000]
    case = _hand_case(lens, budgets)
    rows = case.total_rows()
    g = np.random.default_rng(31)
    pool = np.array([0.0, -0.0, 1.5, -1.5, np.inf, -np.inf, np.nan, 3.25, 1e-38, -1e-38], np.float32)
    sc = g.choice(pool, size=rows).astype(np.float32)
    s0, n0 = case.unit_rows(5, 0, 1)
    sc[s0:s0 + n0] = 2.0
    for seq, h in ((6, 0), (8, 1)):
        s1, n1 = case.unit_rows(seq, 0, h)
        sc[s1:s1 + n1] = g.normal(size=n1).astype(np.float32)
    s2, n2 = case.unit_rows(9, 0, 0)
    sc[s2:s2 + n2] = np.nan
    sc[s2 + g.choice(n2, size=1000, replace=False)] = g.normal(size=1000).astype(np.float32)
    res = gpu_run(case, scores_in=torch.as_tensor(sc, device=DEV))
    check_selection_exact(case, res)
    ostart, b = case.unit_out_rows(5, 0, 1)
    np.testing.assert_array_equal(res["kept"][ostart:ostart + b].cpu().numpy(), np.arange(32767))
    ostart, b = case.unit_out_rows(9, 0, 0)
    assert int(res["kept"][ostart + b - 1]) < n2


def test_select_stream_edge_cases_exact():
    """A batch whose longest unit (35840 keys) takes the streaming select
    (4096 < n <= 35840, keys in per-wave segments): empty, single-key, fully
    kept and budget-0 units, lengths that are not multiples of 64, units far
    shorter than the segments of 8 waves; NaN, signed zeros, infinities and
    denormals; an all-equal unit (the candidate list of the top digit
    overflows, so the lower digits come from sweeps over the unit) and
    normal scores (the lower digits come from the candidate list)."""
    lens = [0, 1, 5, 64, 4097, 35840, 20000, 9999, 12345, 513]
    budgets = [4, 0, 9, 64, 1, 35839, 2, 9998, 6000, 100]
    case = _hand_case(lens, budgets)
    rows = case.total_rows()
    g = np.random.default_rng(29)
    pool = np.array([0.0, -0.0, 1.5, -1.5, np.inf, -np.inf, np.nan, 3.25, 1e-38, -1e-38], np.float32)
    sc = g.choice(pool, size=rows).astype(np.float32)
    s0, n0 = case.unit_rows(5, 0, 1)
    sc[s0:s0 + n0] = 2.0
    for seq, h in ((6, 0), (8, 1), (9, 0)):
        s1, n1 = case.unit_rows(seq, 0, h)
        sc[s1:s1 + n1] = g.normal(size=n1).astype(np.float32)
    res = gpu_run(case, scores_in=torch.as_tensor(sc, device=DEV))
    check_selection_exact(case, res)
    ostart, b = case.unit_out_rows(5, 0, 1)
    np.testing.assert_array_equal(res["kept"][ostart:ostart + b].cpu().numpy(), np.arange(35839))


def test_select_split_edge_cases_exact():
    """A batch whose longest unit (70001 keys) is past what one work-group's
    select holds, so every unit of it takes the split select (tiles of 4096
    keys): empty, single-key, fully kept and budget-0 units next to long
    ones; NaN, signed zeros, infinities and denormals; an all-equal unit
    (ties across every tile boundary) and budgets one below the length."""
    lens = [0, 1, 5, 4096, 4097, 36000, 50000, 70001]
    budgets = [4, 0, 9, 4096, 17, 35999, 1, 70000]
    case = _hand_case(lens, budgets)
    rows = case.total_rows()
    g = np.random.default_rng(71)
    pool = np.array([0.0, -0.0, 1.5, -1.5, np.inf, -np.inf, np.nan, 3.25, 1e-38, -1e-38], np.float32)
    sc = g.choice(pool, size=rows).astype(np.float32)
    s0, n0 = case.unit_rows(5, 0, 1)
    sc[s0:s0 + n0] = 2.0
    s1, n1 = case.unit_rows(6, 0, 0)
    sc[s1:s1 + n1] = g.normal(size=n1).astype(np.float32)
    s2, n2 = case.unit_rows(7, 0, 1)
    sc[s2:s2 + n2] = g.integers(-3, 4, size=n2).astype(np.float32) * 0.5
    res = gpu_run(case, scores_in=torch.as_tensor(sc, device=DEV))
    check_selection_exact(case, res)
    ostart, b = case.unit_out_rows(5, 0, 1)
    np.testing.assert_array_equal(res["kept"][ostart:ostart + b].cpu().numpy(), np.arange(35999))


@pytest.mark.parametrize("n,B", [(35841, 35840), (40000, 1), (131072, 4096), (100000, 50000)])
def test_select_split_many_ties(n, B):
    """Split select on 7 distinct score values: the threshold value spans
    every tile, so each tile's share of the quota comes from the counts of
    the tiles before it."""
    case = _hand_case([n], [B], Hkv=1)
    g = np.random.default_rng(n + B + 1)
    sc = g.integers(-3, 4, size=n).astype(np.float32) * 0.5
    res = gpu_run(case, scores_in=torch.as_tensor(sc, device=DEV))
    check_selection_exact(case, res)


# ---------------------------------------------- full sizes (bench launch)
def _sample(units, k, seed=0):
    g = np.random.default_rng(seed)
    idx = sorted(g.choice(len(units), size=min(k, len(units)), replace=False).tolist())
    return [units[i] for i in idx]


# The five workload configs must not lean on the fp32-resolution floor: it
# is there for degenerate units (spread below the raw scores' resolution),
# which these workloads do not have.
def _assert_no_floor(floors, what):
    above = [f for f in floors if f > 1e-4]
    assert not above, f"{what}: {len(above)} unit(s) need a floor above 1e-4 (max {max(above):.2e})"


@pytest.mark.timeout(900)
def test_long_reasoning_full_size_all_units():
    """32K -> 2048 long-reasoning workload at full size, in the bench's launch:
    scores and (mu, sigma) of all 896 units against the factored oracle (over
    the host's cores), one unit term by term, selection bit-exact on every
    unit, rows on sampled units."""
    case = synth.workload_case("long_reasoning", device=DEV)
    res = gpu_run(case, raw=False, stats=True)
    units = units_of(case)
    _, floors = compare_units_pool(case, res, units)
    _assert_no_floor(floors, "long_reasoning")
    samp = _sample(units, 6, seed=3)
    _compare_units(case, res, samp[:1], factored=False)
    check_selection_exact(case, res, units=units, rows_units=samp)
    check_kept_near_threshold(case, res, samp)


@pytest.mark.timeout(900)
def test_decode_window_full_size_all_units():
    """Decode-window trigger at full size (64 sequences x 32 layers x 8 KV
    heads, 3200 keys each): all 16384 units against the factored oracle,
    selection bit-exact on 2000 sampled units."""
    case = synth.workload_case("decode_window", device=DEV)
    res = gpu_run(case, raw=False, stats=True)
    units = units_of(case)
    _, floors = compare_units_pool(case, res, units)
    _assert_no_floor(floors, "decode_window")
    samp = _sample(units, 6, seed=2)
    check_kept_near_threshold(case, res, samp)
    check_selection_exact(case, res, units=_sample(units, 2000, seed=5), rows_units=samp)


@pytest.mark.timeout(900)
def test_ragged_full_layer_all_units():
    """Ragged batch (256 sequences of 2048..16384 keys, one layer of 8 KV
    heads): all units against the factored oracle, selection bit-exact on
    every unit."""
    case = synth.workload_case("ragged", device=DEV)
    res = gpu_run(case, raw=False, stats=True)
    units = units_of(case)
    _, floors = compare_units_pool(case, res, units)
    _assert_no_floor(floors, "ragged")
    samp = _sample(units, 6, seed=4)
    check_kept_near_threshold(case, res, samp)
    check_selection_exact(case, res, units=units, rows_units=samp)


@pytest.mark.timeout(600)
def test_stress_ties_full_size():
    case = synth.workload_case("stress_ties", device=DEV)
    res = gpu_run(case, raw=False, stats=True)
    units = units_of(case)
    _, floors = _compare_units(case, res, units, factored=True, floors=True)
    _assert_no_floor(floors, "stress_ties")
    check_selection_exact(case, res, units=units, rows_units=units[:2])
    check_kept_near_threshold(case, res, units)
    sc = res["scores"].cpu().numpy()
    for (s, l, g) in units:
        start, n = case.unit_rows(s, l, g)
        u = sc[start:start + n].reshape(-1, 128)
        assert np.array_equal(u[:, 64:].view(np.uint32), u[:, :64].view(np.uint32))


@pytest.mark.timeout(600)
def test_unit_past_fused_chunk_cap():
    """A unit of more than 384 fused chunks (here 394216 keys at G = 7, chunks
    of at most 1024 keys) is scored by the generic path; scores against the
    oracle, selection exact."""
    shape = synth.Shape(128, 7, 1, 1)
    case = synth.build_case("long_unit", shape, [1024 * 384 + 1000], [4096], device=DEV, seed=11)
    res = gpu_run(case, raw=False, stats=True)
    units = units_of(case)
    _compare_units(case, res, units, factored=True)
    check_selection_exact(case, res, units=units, rows_units=units)


def _to_host(res):
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in res.items()}


def _to_device(case):
    import dataclasses
    mv = {f: getattr(case, f).to(DEV) for f in ("k", "v", "k_pos", "q_centre", "q_absmean", "q_R")
          if getattr(case, f) is not None}
    return dataclasses.replace(case, **mv)


@pytest.mark.parametrize("S", [3000, 8192])
def test_many_tiny_sequences(S):
    """Thousands of sequences of 0..40 keys (up to the 8192 a call takes;
    most units a single partial tile, many empty or fully kept): scores
    against the oracle on every unit, selection and rows exact."""
    g = np.random.default_rng(17 + S)
    lens = g.integers(0, 41, size=S)
    lens[g.choice(S, S // 10, replace=False)] = 0
    budgets = g.integers(0, 51, size=S)
    shape = synth.Shape(64, 4, 2, 1)
    # the checks read the host copy (thousands of units: no per-unit device reads)
    host = synth.build_case("tiny", shape, lens.tolist(), budgets.tolist(), seed=17)
    res = _to_host(gpu_run(_to_device(host), raw=True, stats=True))
    units = units_of(host)
    _compare_units(host, res, units if S <= 3000 else units[::5], factored=True)
    check_selection_exact(host, res)


def test_many_tiny_sequences_max_offsets():
    """The max-over-offsets path on the same kind of batch (d = 128)."""
    from harness import gpu_score_offsets
    g = np.random.default_rng(19)
    S = 1500
    lens = g.integers(0, 70, size=S)
    shape = synth.Shape(128, 8, 2, 1)
    case = synth.build_case("tiny_max", shape, lens.tolist(), [1] * S, seed=19)
    offs = [1.0, 16.0, 256.0, 4096.0]
    res = _to_host(gpu_score_offsets(_to_device(case), offs, "max", raw=True, stats=True))
    sc = res["scores"].cpu().numpy()
    for (s, l, gg) in units_of(case)[::7]:
        if case.seq_len(s) == 0:
            continue
        start, n, ref, S, _, sigma = oracle_unit(case, s, l, gg, factored=True, offsets=offs,
                                                 reduce="max")
        check_scores(sc[start:start + n], ref, f"tiny max unit {(s, l, gg)}", z_floor(S, sigma))


@pytest.mark.parametrize("seed", range(12))
def test_calibrate_random(seed):
    """Seeded random calibration shapes: any head_dim multiple of 8, query
    heads, layers, sample counts (ragged against the 256-sample chunks),
    post-RoPE or pre-RoPE samples, either RoPE layout."""
    import rope_aware_key_amd as R
    g = np.random.default_rng([94, seed])
    d = int(g.integers(1, 33)) * 8
    Hq, L, N = int(g.integers(1, 12)), int(g.integers(1, 3)), int(g.integers(1, 1300))
    layout = "half" if g.random() < 0.5 else "interleaved"
    post = g.random() < 0.7
    torch.manual_seed(seed)
    q = (torch.randn(L, N, Hq, d, device=DEV) * 0.7 + 0.5).to(torch.bfloat16).view(torch.int16)
    q_pos = torch.as_tensor(g.integers(0, 40000, size=N), dtype=torch.int32, device=DEV) if post else None
    sh = R.make_shape(d, Hq, 1, L, rope_layout=layout)
    c = torch.empty(L, Hq, d // 2, 2, device=DEV)
    a = torch.empty(L, Hq, d // 2, device=DEV)
    r = torch.empty(L, Hq, d // 2, device=DEV)
    R.tri_calibrate(sh, q, q_pos, N, c, a, r)
    torch.cuda.synchronize()
    qq = O.bf16_bits_to_f64(q.cpu().numpy().view(np.uint16))
    om = O.rope_omega(d, 1e4)
    qp = None if q_pos is None else q_pos.cpu().numpy()
    for l in range(L):
        centre, absmean, Rr = O.calibrate(qq[l], qp, om, layout=layout)
        np.testing.assert_allclose(c[l, ..., 0].cpu().numpy(), centre.real, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(c[l, ..., 1].cpu().numpy(), centre.imag, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(a[l].cpu().numpy(), absmean, rtol=1e-5)
        np.testing.assert_allclose(r[l].cpu().numpy(), Rr, rtol=1e-5, atol=1e-6)

