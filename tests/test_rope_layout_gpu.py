"""Half-split RoPE layout (rope_layout = TRI_ROPE_HALF_SPLIT) against the oracle.

Every case is a synthetic interleaved case with the columns of its keys
(and calibration queries) permuted to the half layout; the oracle scores
the permuted keys with layout="half".  Bars as for the interleaved layout:
scores |gpu - ref| <= 1e-4 * max(1, |ref|), raw S~ within 1e-4 of
max(|S~|, sigma), selection bit-exact on the GPU's own scores, r within
2e-5.  head_dim % 64 == 0 takes the MFMA kernels; other head_dims take the
VALU path (tri_score) or are refused (the max over offsets).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import (z_floor, check_raw, check_scores, check_selection_exact, gpu_calibrate, gpu_run,
                     gpu_score_offsets, half_split, oracle_unit, shape_of, units_of)
from synth.cases import _calibration_queries

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _compare(case, res, units, factored=True, offsets=None, reduce="mean"):
    scores = res["scores"].cpu().numpy()
    raw = res["raw"].cpu().numpy() if res.get("raw") is not None else None
    hs = res["head_stats"].cpu().numpy() if res.get("head_stats") is not None else None
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    for (s, l, g) in units:
        if case.seq_len(s) == 0:
            continue
        start, n, ref, S, mu, sigma = oracle_unit(case, s, l, g, factored=factored,
                                                  offsets=offsets, reduce=reduce)
        check_scores(scores[start:start + n], ref, f"half unit {(s, l, g)}", z_floor(S, sigma))
        if raw is not None:
            check_raw(raw[start:start + n], S, sigma, f"half raw unit {(s, l, g)}")
        if hs is not None:
            u = (s * L + l) * H + g
            np.testing.assert_allclose(hs[u, :, 0], mu, rtol=0, atol=1e-5 * max(np.max(sigma), np.max(np.abs(S))))
            np.testing.assert_allclose(hs[u, :, 1], sigma, rtol=1e-5, atol=1e-5 * np.max(np.abs(S)))


@pytest.mark.parametrize("d,G", [(128, 4), (64, 7), (256, 2), (192, 3), (96, 4), (24, 2)])
def test_half_split_scores_and_selection(d, G):
    """MFMA path for d in {64, 128, 192, 256}, VALU path for 96 and 24;
    a ragged batch with an empty sequence and a ragged tail."""
    shape = synth.Shape(d, 2 * G, 2, 2)
    base = synth.build_case("half", shape, [300, 0, 1000, 2100], [128, 5, 1000, 3000],
                            device=DEV, seed=d + G)
    case = half_split(base)
    res = gpu_run(case, raw=True, stats=True)
    units = units_of(case)
    _compare(case, res, units, factored=True)
    _compare(case, res, units[:2], factored=False)
    check_selection_exact(case, res)


def test_half_split_scores_follow_the_layout():
    """The half-split scores of the permuted keys track the interleaved
    scores of the original keys (same math, other storage), and reading
    half-split keys as interleaved would not."""
    shape = synth.Shape(128, 8, 2, 1)
    base = synth.build_case("half_vs", shape, [1500], [100], device=DEV, seed=4)
    a = gpu_run(base, raw=False, stats=False, compact=False)["scores"].cpu().numpy()
    b = gpu_run(half_split(base), raw=False, stats=False, compact=False)["scores"].cpu().numpy()
    np.testing.assert_allclose(b, a, rtol=0, atol=2e-4 * max(1.0, np.abs(a).max()))
    wrong = half_split(base)
    wrong.meta = dict(wrong.meta, rope_layout="interleaved")
    c = gpu_run(wrong, raw=False, stats=False, compact=False)["scores"].cpu().numpy()
    assert np.max(np.abs(c - a)) > 1e-2


@pytest.mark.parametrize("reduce", ["mean", "max"])
@pytest.mark.parametrize("d,G", [(128, 7), (64, 4)])
def test_half_split_offsets(reduce, d, G):
    offs = [float(x) for x in range(1, 129, 8)]
    shape = synth.Shape(d, 2 * G, 2, 1)
    case = half_split(synth.build_case("half_off", shape, [700, 64, 2049], [1, 1, 1],
                                       device=DEV, seed=d * G))
    res = gpu_score_offsets(case, offs, reduce)
    _compare(case, res, units_of(case), offsets=offs, reduce=reduce)


def test_half_split_max_refused_for_odd_steps():
    import rope_aware_key_amd as R
    sh = R.make_shape(96, 4, 2, 1, rope_layout="half")
    assert R.tri_workspace_bytes_offsets(sh, np.array([0, 8]), 3, "max") == 0


def test_half_split_calibration():
    """Per-band sums do not depend on where the parts are stored: the
    half-split statistics equal the interleaved ones bit for bit, and the
    oracle's within the calibration bar."""
    base = synth.workload_case("smallest", device=DEV, calib_samples=3000)
    case = half_split(base)
    gpu_calibrate(base)
    gpu_calibrate(case)
    for a, b in ((base.q_centre, case.q_centre), (base.q_absmean, case.q_absmean),
                 (base.q_R, case.q_R)):
        assert torch.equal(a, b)
    q = O.bf16_bits_to_f64(case.calib_q[0].cpu().numpy().view(np.uint16))
    om = O.rope_omega(128, 1e4)
    centre, absmean, Rr = O.calibrate(q, case.calib_pos.cpu().numpy(), om, layout="half")
    qc = case.q_centre[0].cpu().double().numpy()
    np.testing.assert_allclose(qc[..., 0], centre.real, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(qc[..., 1], centre.imag, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(case.q_absmean[0].cpu().double().numpy(), absmean, rtol=1e-5)
    np.testing.assert_allclose(case.q_R[0].cpu().double().numpy(), Rr, rtol=1e-5)


@pytest.mark.parametrize("d,G", [(128, 4), (96, 2)])
def test_half_split_trig_correlation(d, G):
    import rope_aware_key_amd as R
    shape = synth.Shape(d, 2 * G, 2, 1)
    n_q, n_k = 70, 150
    q, q_pos = _calibration_queries(shape, n_q, DEV, 7, R_Q=0.9)
    case = half_split(synth.build_case("diag_half", shape, (n_k,), (1,), device=DEV, seed=7,
                                       with_values=False))
    perm = torch.as_tensor(np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)]), device=DEV)
    qh = q[..., perm].contiguous()
    L, Hq, Hkv = 1, 2 * G, 2
    om = O.rope_omega(d, shape.rope_theta)
    qb = O.bf16_bits_to_f64(qh.cpu().numpy().view(np.uint16))
    qp = q_pos.cpu().numpy().astype(np.float64)
    c, _, _ = O.calibrate(qb[0], qp, om, layout="half")
    centre = np.stack([c.real, c.imag], axis=-1).astype(np.float32)[None]
    sh = shape_of(case)
    ws = torch.empty(R.tri_trig_correlation_workspace_bytes(sh, n_q), dtype=torch.uint8, device=DEV)
    r = torch.full((L, Hq), float("nan"), dtype=torch.float64, device=DEV)
    R.tri_trig_correlation(sh, qh, q_pos, n_q, case.k, case.k_pos, n_k,
                           torch.as_tensor(centre, device=DEV), r, workspace=ws)
    torch.cuda.synchronize()
    r = r.cpu().numpy()
    kb = O.bf16_bits_to_f64(case.k.cpu().numpy().view(np.uint16))
    kp = case.k_pos.cpu().numpy().astype(np.float64)
    for h in range(Hq):
        u = h // G
        cc = centre[0, h, :, 0].astype(np.float64) + 1j * centre[0, h, :, 1].astype(np.float64)
        ref = O.trig_reconstruction_r(qb[0, :, h, :], qp, kb[u * n_k:(u + 1) * n_k],
                                      kp[u * n_k:(u + 1) * n_k], cc, om, layout="half")
        assert abs(r[0, h] - ref) <= 2e-5, (h, r[0, h], ref)


@pytest.mark.timeout(600)
def test_half_split_long_reasoning_full_size():
    """The 32K -> 2048 workload stored half split: sampled units against the
    oracle, selection bit-exact on every unit."""
    case = half_split(synth.workload_case("long_reasoning", device=DEV))
    res = gpu_run(case, raw=False, stats=True)
    units = units_of(case)
    g = np.random.default_rng(9)
    samp = [units[i] for i in sorted(g.choice(len(units), 4, replace=False))]
    _compare(case, res, samp, factored=True)
    check_selection_exact(case, res, units=units, rows_units=samp[:2])
