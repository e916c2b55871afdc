"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Each test ties the oracle to something other than itself: a hand-derived
closed form (tests/golden/hand_cases.json), an independent computation path
(the explicit RoPE dot product instead of the cosine series), an invariant,
or brute-force enumeration.  None of these needs a GPU.
"""
import json
import math
import os

import itertools

import numpy as np
import pytest

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def _direct_logit(q_pre, p_q, k_post):
    """Attention logit the plain way: rotate the query to p_q, dot with the
    stored (already rotated) key.  No cosine series involved."""
    om = O.rope_omega(q_pre.shape[-1], _direct_logit.theta)
    return O.rope_rotate(q_pre, p_q, om) @ k_post


_direct_logit.theta = 10000.0


# ---------------------------------------------------------------- RoPE ----
def test_omega_closed_forms():
    g = GOLD["omega_closed_forms"]
    om = O.rope_omega(g["d"], g["theta"])
    for f, w in zip(g["f"], g["omega"]):
        assert om[f] == pytest.approx(w, rel=1e-14)


def test_rope_quarter_turn_matches_printed_matrix():
    g = GOLD["rope_quarter_turn"]
    om = O.rope_omega(g["d"], g["theta"])
    for x, y in zip(g["inputs"], g["outputs"]):
        out = O.rope_rotate(np.array(x), g["pos"], om)
        np.testing.assert_allclose(out, y, atol=1e-15)


def test_rope_group_properties():
    rng = np.random.default_rng(1)
    om = O.rope_omega(64, 1e4)
    x = rng.normal(size=(5, 64))
    p1, p2 = 1234.0, 98765.0
    a = O.rope_rotate(O.rope_rotate(x, p1, om), p2, om)
    b = O.rope_rotate(x, p1 + p2, om)
    np.testing.assert_allclose(a, b, atol=1e-11)
    np.testing.assert_allclose(O.rope_derotate(O.rope_rotate(x, p2, om), p2, om), x, atol=1e-11)
    # norms of every band are preserved
    np.testing.assert_allclose(np.abs(O.bands(O.rope_rotate(x, p2, om))), np.abs(O.bands(x)), rtol=1e-13)


def test_rope_relative_position_property():
    """q_i^T k_j depends only on i - j (tutorial page, RoPE paragraph)."""
    rng = np.random.default_rng(2)
    om = O.rope_omega(128, 1e4)
    q, k = rng.normal(size=128), rng.normal(size=128)
    a = O.rope_rotate(q, 5000.0, om) @ O.rope_rotate(k, 1000.0, om)
    b = O.rope_rotate(q, 104000.0, om) @ O.rope_rotate(k, 100000.0, om)
    assert a == pytest.approx(b, rel=1e-9, abs=1e-9)


# ---------------------------------------------------- logit decomposition ----
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_logit_decomposition_vs_direct_dot(seed):
    rng = np.random.default_rng(seed)
    d = 128
    om = O.rope_omega(d, 1e4)
    q = rng.normal(size=(50, d))
    k = rng.normal(size=(50, d))
    pq = rng.integers(0, 200000, size=50).astype(float)
    pk = rng.integers(0, 200000, size=50).astype(float)
    direct = np.einsum("nd,nd->n", O.rope_rotate(q, pq, om), O.rope_rotate(k, pk, om))
    series = O.logit_decomposed(q, k, pq - pk, om)
    scale = np.sum(np.abs(O.bands(q)) * np.abs(O.bands(k)), axis=1)
    assert np.max(np.abs(direct - series) / scale) < 1e-12


# ------------------------------------------------------------- S_trig ----
def _unit(rng, n, d, p_q_max=70000):
    om = O.rope_omega(d, 1e4)
    pos = np.sort(rng.choice(p_q_max - 1, size=n, replace=False)).astype(float)
    k_pre = rng.normal(size=(n, d)) + 1.5
    k_post = O.rope_rotate(k_pre, pos, om)
    return om, pos, k_post


def test_strig_equals_mean_logit_when_queries_equal_centre():
    """Every query equals its centre: R_f = 1, S_norm = 0, and the averaged
    score equals the mean over D of the direct logit at distance Delta + delta."""
    rng = np.random.default_rng(3)
    d, n = 32, 40
    om, pos, k_post = _unit(rng, n, d)
    c = rng.normal(size=d)
    qpos = np.arange(16, dtype=float) * 37.0
    q_post = O.rope_rotate(np.tile(c, (16, 1))[:, None, :], qpos[:, None], om)  # [N,1,d]
    centre, absmean, R = O.calibrate(q_post, qpos, om)
    np.testing.assert_allclose(R, 1.0, atol=1e-13)
    p_q = 70000.0
    S, s_trig, s_norm = O.score_terms(k_post, pos, p_q, centre, absmean, R, om)
    assert np.max(np.abs(s_norm)) < 1e-10
    ref = np.mean([_direct_logit(c, p_q + dl, k_post.T) for dl in O.OFFSETS], axis=0)
    assert np.max(np.abs(S[0] - ref)) < 1e-11 * np.max(np.abs(ref))


def test_score_linearity_for_any_concentration():
    """S_trig is linear in the query: the averaged trig term equals the mean
    over the calibration set and over D of the direct logit, for any R; and
    S_norm = sum_f (E|q_f| - |E q_f|) |k_f|."""
    rng = np.random.default_rng(4)
    d, n, N = 32, 30, 200
    om, pos, k_post = _unit(rng, n, d)
    q_pre = rng.normal(size=(N, d)) * 0.8 + rng.normal(size=d)
    qpos = rng.integers(0, 5000, size=N).astype(float)
    q_post = O.rope_rotate(q_pre[:, None, :], qpos[:, None], om)
    centre, absmean, R = O.calibrate(q_post, qpos, om)
    assert np.all(R < 1.0) and np.all(R > 0.0)
    p_q = 70000.0
    S, s_trig, s_norm = O.score_terms(k_post, pos, p_q, centre, absmean, R, om)
    ref_trig = np.zeros(n)
    for dl in O.OFFSETS:
        ref_trig += np.mean(O.rope_rotate(q_pre, p_q + dl, om) @ k_post.T, axis=0)
    ref_trig /= len(O.OFFSETS)
    assert np.max(np.abs(s_trig[0] - ref_trig)) < 1e-11 * np.max(np.abs(ref_trig))
    qf = q_pre[:, 0::2] + 1j * q_pre[:, 1::2]
    k_abs = np.abs(k_post[:, 0::2] + 1j * k_post[:, 1::2])   # rotation keeps |k_f|
    gap = np.mean(np.abs(qf), axis=0) - np.abs(np.mean(qf, axis=0))
    ref_norm = k_abs @ gap
    np.testing.assert_allclose(s_norm[0], ref_norm, rtol=1e-11)


@pytest.mark.parametrize("case", ["offset_mean_omega_pi", "offset_mean_omega_half_pi"])
def test_offset_average_closed_form(case):
    """d = 4 with theta chosen so omega_1 is pi or pi/2: the 17-offset mean has
    a closed form, which pins the offset set (2^0..2^16, 17 items)."""
    g = GOLD[case]
    omega1 = math.pi if case.endswith("_pi") and "half" not in case else math.pi / 2
    theta = omega1 ** -2.0
    om = O.rope_omega(4, theta)
    assert om[1] == pytest.approx(omega1, rel=1e-14)
    rng = np.random.default_rng(5)
    n = 12
    pos = np.arange(n, dtype=float) * 3.0
    k_pre = np.zeros((n, 4))
    k_pre[:, 2:] = rng.normal(size=(n, 2))
    k_post = O.rope_rotate(k_pre, pos, om)
    cq = np.array([0.0, 0.0, 0.7, -1.3])
    centre = O.bands(cq)[None, :]
    absmean = np.abs(centre) * 1.25
    R = np.abs(centre) / np.where(absmean > 0, absmean, 1.0)
    R[absmean == 0] = 1.0
    p_q = 1000.0
    _, s_trig, _ = O.score_terms(k_post, pos, p_q, centre, absmean, R, om)
    kf = O.bands(k_pre)[:, 1]
    qf = O.bands(cq)[1]
    psi = omega1 * (p_q - pos) + np.angle(qf) - np.angle(kf)
    amp = abs(qf) * np.abs(kf)
    if "half" in case:
        expect = amp * (14.0 * np.cos(psi) - np.sin(psi)) / 17.0
        C = O.offset_phasor_mean(om)[1]
        # omega_1 * 2^16 carries ~1e-11 rad of fp64 rounding of pi
        assert C.real == pytest.approx(g["C_re"], abs=1e-10)
        assert C.imag == pytest.approx(g["C_im"], abs=1e-10)
    else:
        expect = g["ratio"] * amp * np.cos(psi)
    np.testing.assert_allclose(s_trig[0], expect, atol=1e-9 * np.max(amp))


def test_factored_equals_term_by_term():
    rng = np.random.default_rng(6)
    d, n, G = 128, 64, 3
    om, pos, k_post = _unit(rng, n, d, p_q_max=131072)
    F = d // 2
    centre = rng.uniform(0.5, 2, size=(G, F)) * np.exp(1j * rng.uniform(0, 2 * np.pi, size=(G, F)))
    R = rng.uniform(0.3, 0.99, size=(G, F))
    absmean = np.abs(centre) / R
    p_q = 131072.0
    S_terms = O.score_terms(k_post, pos, p_q, centre, absmean, R, om)[0]
    S_fact = O.score_factored(k_post, p_q, centre, absmean, R, om)
    assert np.max(np.abs(S_terms - S_fact)) < 1e-12 * np.max(np.abs(S_terms))


def test_offset_phasor_limits():
    om = np.array([1e-12, 1e-3, 0.1, 1.0])
    C = O.offset_phasor_mean(om)
    assert np.all(np.abs(C) <= 1.0 + 1e-15)
    assert abs(C[0] - 1.0) < 1e-6


def test_key_position_cancels():
    """The same stored (post-RoPE) key at two positions scores the same, and
    shifting every position and p_q by t (keys re-rotated) changes nothing."""
    rng = np.random.default_rng(7)
    d, n, G = 64, 20, 2
    om, pos, k_post = _unit(rng, n, d)
    F = d // 2
    centre = rng.normal(size=(G, F)) + 1j * rng.normal(size=(G, F))
    R = rng.uniform(0.5, 1.0, size=(G, F))
    absmean = np.abs(centre) / R
    k2 = np.concatenate([k_post, k_post[:5]])
    pos2 = np.concatenate([pos, pos[:5] + 77.0])
    S = O.score_terms(k2, pos2, 80000.0, centre, absmean, R, om)[0]
    np.testing.assert_allclose(S[:, n:], S[:, :5], rtol=1e-11, atol=1e-11)
    k_pre = O.rope_derotate(k_post, pos, om)
    t = 12345.0
    S_a = O.score_terms(k_post, pos, 80000.0, centre, absmean, R, om)[0]
    S_b = O.score_terms(O.rope_rotate(k_pre, pos + t, om), pos + t, 80000.0 + t,
                        centre, absmean, R, om)[0]
    np.testing.assert_allclose(S_a, S_b, rtol=1e-9, atol=1e-9)


# --------------------------------------------------------- S_norm / R ----
def test_antipodal_queries_zero_trig():
    """Samples (q, -q) at the same position: E[q_f] = 0, R_f = 0, S_trig = 0
    and S = sum_f E|q_f| |k_f|."""
    rng = np.random.default_rng(8)
    d = 16
    om = O.rope_omega(d, 1e4)
    q = rng.normal(size=(10, d))
    qq = np.concatenate([q, -q])[:, None, :]
    qpos = np.concatenate([np.arange(10.0), np.arange(10.0)])
    centre, absmean, R = O.calibrate(O.rope_rotate(qq, qpos[:, None], om), qpos, om)
    assert np.max(np.abs(centre)) < 1e-13
    np.testing.assert_allclose(R, 0.0, atol=1e-13)
    _, pos, k_post = _unit(rng, 8, d)
    S, s_trig, s_norm = O.score_terms(k_post, pos, 9000.0, centre, absmean, R, om)
    assert np.max(np.abs(s_trig)) < 1e-12
    kabs = np.abs(O.bands(k_post))
    np.testing.assert_allclose(S[0], kabs @ absmean[0], rtol=1e-12)


def test_calibration_hand_example():
    g = GOLD["calibration_two_samples"]
    om = O.rope_omega(2, g["theta"])
    q_post = np.array([[[3.0, 4.0]], [[-5.0 * math.sin(1.0), 5.0 * math.cos(1.0)]]])
    centre, absmean, R = O.calibrate(q_post, np.array([0.0, 1.0]), om)
    assert centre[0, 0].real == pytest.approx(g["centre"][0], abs=1e-14)
    assert centre[0, 0].imag == pytest.approx(g["centre"][1], abs=1e-14)
    assert absmean[0, 0] == pytest.approx(g["absmean"], rel=1e-15)
    assert R[0, 0] == pytest.approx(g["R"], rel=1e-14)


def test_calibration_identical_samples():
    rng = np.random.default_rng(9)
    d = 8
    om = O.rope_omega(d, 1e4)
    c = rng.normal(size=d)
    qpos = np.arange(7, dtype=float) * 1001
    q_post = O.rope_rotate(np.tile(c, (7, 1))[:, None, :], qpos[:, None], om)
    centre, absmean, R = O.calibrate(q_post, qpos, om)
    np.testing.assert_allclose(R, 1.0, atol=1e-12)
    np.testing.assert_allclose(absmean, np.abs(centre), rtol=1e-12)
    np.testing.assert_allclose(centre[0], O.bands(c), atol=1e-12)
    # pre-RoPE samples (q_pos None) skip the de-rotation
    c2, a2, R2 = O.calibrate(np.tile(c, (3, 1))[:, None, :], None, om)
    np.testing.assert_allclose(c2[0], O.bands(c), atol=1e-15)


def test_calibration_zero_band_reads_R_one():
    q = np.zeros((4, 1, 4))
    q[:, 0, 2:] = [1.0, 0.5]
    c, a, R = O.calibrate(q, None, O.rope_omega(4, 1e4))
    assert R[0, 0] == 1.0 and a[0, 0] == 0.0


# ---------------------------------------------------------- z and max ----
def test_zscore_hand_example():
    g = GOLD["zscore_1234"]
    z, mu, sigma = O.zscore_rows(np.array([g["raw"]]))
    np.testing.assert_allclose(z[0], g["z"], rtol=1e-14)


def test_zscore_invariants_and_max():
    rng = np.random.default_rng(10)
    S = rng.normal(size=(5, 300)) * rng.uniform(0.1, 5, size=(5, 1)) + rng.normal(size=(5, 1)) * 10
    z, mu, sigma = O.zscore_rows(S)
    np.testing.assert_allclose(z.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(np.sqrt((z ** 2).mean(axis=1)), 1.0, rtol=1e-12)
    z2, _, _ = O.zscore_rows(S * 3.7 + 11.0)
    np.testing.assert_allclose(z2, z, atol=1e-11)
    m = O.gqa_max(z)
    assert np.all(m[None, :] >= z - 0.0)
    assert np.all(np.any(z == m[None, :], axis=0))
    z1, _, _ = O.zscore_rows(S[:1])
    np.testing.assert_array_equal(O.gqa_max(z1), z1[0])
    zc, _, sc = O.zscore_rows(np.full((1, 9), 4.2))
    assert sc[0] == 0.0 and np.all(zc == 0.0)


def test_unit_scores_scale_invariance():
    """Scaling (E[q], E|q|) of every head by c > 0 leaves the final scores unchanged."""
    rng = np.random.default_rng(11)
    d, n, G = 32, 50, 4
    om, pos, k_post = _unit(rng, n, d)
    F = d // 2
    centre = rng.normal(size=(G, F)) + 1j * rng.normal(size=(G, F))
    R = rng.uniform(0.5, 1.0, size=(G, F))
    absmean = np.abs(centre) / R
    a = O.unit_scores(k_post, pos, 1e5, centre, absmean, R, om)[0]
    b = O.unit_scores(k_post, pos, 1e5, centre * 2.5, absmean * 2.5, R, om)[0]
    np.testing.assert_allclose(a, b, atol=1e-10)


# ------------------------------------------------------------- select ----
@pytest.mark.parametrize("seed", range(12))
def test_select_matches_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 10))
    pool = np.array([0.5, -0.5, 1.0, 0.0, -0.0, np.inf, -np.inf, np.nan, 2.0], dtype=np.float32)
    s = rng.choice(pool, size=n) if seed % 2 else rng.normal(size=n).astype(np.float32)
    for B in range(0, n + 2):
        np.testing.assert_array_equal(O.select_topb(s, B), O.select_topb_bruteforce(s, B))


def test_select_edge_cases():
    s = np.full(10, 3.0, dtype=np.float32)
    np.testing.assert_array_equal(O.select_topb(s, 4), [0, 1, 2, 3])
    np.testing.assert_array_equal(O.select_topb(s, 50), np.arange(10))
    assert O.select_topb(s, 0).size == 0
    assert O.select_topb(np.zeros(0, np.float32), 5).size == 0
    s = np.array([0.0, -0.0, 0.0, -0.0], dtype=np.float32)
    np.testing.assert_array_equal(O.select_topb(s, 2), [0, 1])
    s = np.array([np.nan, -np.inf, np.nan, 1.0], dtype=np.float32)
    np.testing.assert_array_equal(O.select_topb(s, 2), [1, 3])
    np.testing.assert_array_equal(O.select_topb(s, 3), [0, 1, 3])


def test_select_permutation_invariance():
    rng = np.random.default_rng(12)
    s = rng.normal(size=200)
    perm = rng.permutation(200)
    a = set(O.select_topb(s, 37).tolist())
    b = set(perm[O.select_topb(s[perm], 37)].tolist())
    assert a == b


def test_compact_rows_bytes():
    rng = np.random.default_rng(13)
    rows = rng.integers(0, 65535, size=(20, 8), dtype=np.uint16)
    kept = O.select_topb(rng.normal(size=20), 7)
    out = O.compact_rows(rows, kept)
    assert np.all(np.diff(kept) > 0)
    for j, i in enumerate(kept):
        assert out[j].tobytes() == rows[i].tobytes()


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0x4049], dtype=np.uint16)
    v = O.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 0.0 and np.signbit(v[3])
    assert np.isinf(v[4]) and v[5] == 3.140625


def test_packed_unit_rows():
    cu = np.array([0, 5, 12])
    assert O.unit_rows(cu, 2, 3, 0, 1, 2) == ((1 * 3 + 2) * 5, 5)
    assert O.unit_rows(cu, 2, 3, 1, 0, 1) == (2 * 3 * 5 + 1 * 7, 7)
    assert O.out_rows(cu, [3, 10], 2, 3, 1, 1, 0) == (2 * 3 * 3 + 1 * 3 * 7, 7)


# ------------------------------------------------ offset-set variants ----
LINEAR_OFFSETS = tuple(float(x) for x in range(1, 129, 8))       # 16 evenly spaced
SHORT_OFFSETS = tuple(float(2 ** m) for m in range(9))            # max distance 256


@pytest.mark.parametrize("offsets", [O.OFFSETS, LINEAR_OFFSETS, SHORT_OFFSETS, (5.0,)])
def test_max_over_offsets_equals_max_logit_when_queries_equal_centre(offsets):
    """Every query equals its centre (R = 1, S_norm = 0): the max-reduced score
    is the largest direct RoPE logit over the offsets (q rotated to
    p_q + delta, dotted with the stored key), for any offset set."""
    rng = np.random.default_rng(31)
    d, n = 32, 40
    om, pos, k_post = _unit(rng, n, d)
    c = rng.normal(size=d)
    qpos = np.arange(16, dtype=float) * 37.0
    q_post = O.rope_rotate(np.tile(c, (16, 1))[:, None, :], qpos[:, None], om)
    centre, absmean, R = O.calibrate(q_post, qpos, om)
    p_q = 70000.0
    S, s_trig, s_norm = O.score_terms(k_post, pos, p_q, centre, absmean, R, om, offsets, "max")
    assert np.max(np.abs(s_norm)) < 1e-10
    ref = np.max([_direct_logit(c, p_q + dl, k_post.T) for dl in offsets], axis=0)
    assert np.max(np.abs(S[0] - ref)) < 1e-11 * np.max(np.abs(ref))


@pytest.mark.parametrize("offsets", [LINEAR_OFFSETS, SHORT_OFFSETS])
def test_mean_over_other_offset_sets_is_mean_logit(offsets):
    """The mean over any offset set equals the mean over the calibration set
    and over that set of direct logits (linearity in q), the same pin as the
    default set with another D."""
    rng = np.random.default_rng(32)
    d, n, N = 32, 30, 100
    om, pos, k_post = _unit(rng, n, d)
    q_pre = rng.normal(size=(N, d)) * 0.8 + rng.normal(size=d)
    qpos = rng.integers(0, 5000, size=N).astype(float)
    q_post = O.rope_rotate(q_pre[:, None, :], qpos[:, None], om)
    centre, absmean, R = O.calibrate(q_post, qpos, om)
    p_q = 70000.0
    _, s_trig, _ = O.score_terms(k_post, pos, p_q, centre, absmean, R, om, offsets, "mean")
    ref = np.mean([np.mean(O.rope_rotate(q_pre, p_q + dl, om) @ k_post.T, axis=0)
                   for dl in offsets], axis=0)
    assert np.max(np.abs(s_trig[0] - ref)) < 1e-11 * np.max(np.abs(ref))


@pytest.mark.parametrize("reduce", ["mean", "max"])
@pytest.mark.parametrize("offsets", [O.OFFSETS, LINEAR_OFFSETS])
def test_factored_equals_term_by_term_for_offset_variants(reduce, offsets):
    rng = np.random.default_rng(33)
    d, n, G = 64, 48, 3
    om, pos, k_post = _unit(rng, n, d, p_q_max=131072)
    F = d // 2
    centre = rng.uniform(0.5, 2, size=(G, F)) * np.exp(1j * rng.uniform(0, 2 * np.pi, size=(G, F)))
    R = rng.uniform(0.3, 0.99, size=(G, F))
    absmean = np.abs(centre) / R
    p_q = 131072.0
    S_terms = O.score_terms(k_post, pos, p_q, centre, absmean, R, om, offsets, reduce)[0]
    S_fact = O.score_factored(k_post, p_q, centre, absmean, R, om, offsets, reduce)
    assert np.max(np.abs(S_terms - S_fact)) < 1e-12 * np.max(np.abs(S_terms))


def test_max_reduction_invariants():
    """max over D >= mean over D key by key; one offset makes them equal;
    repeating offsets changes neither (the GPU pads with repeats)."""
    rng = np.random.default_rng(34)
    d, n, G = 32, 25, 2
    om, pos, k_post = _unit(rng, n, d)
    F = d // 2
    centre = rng.normal(size=(G, F)) + 1j * rng.normal(size=(G, F))
    R = rng.uniform(0.2, 0.9, size=(G, F))
    absmean = np.abs(centre) / R
    p_q = 9000.0
    mx = O.score_factored(k_post, p_q, centre, absmean, R, om, O.OFFSETS, "max")
    mn = O.score_factored(k_post, p_q, centre, absmean, R, om, O.OFFSETS, "mean")
    assert np.all(mx >= mn - 1e-12 * np.max(np.abs(mn)))
    one_max = O.score_factored(k_post, p_q, centre, absmean, R, om, (64.0,), "max")
    one_mean = O.score_factored(k_post, p_q, centre, absmean, R, om, (64.0,), "mean")
    np.testing.assert_allclose(one_max, one_mean, rtol=1e-12, atol=1e-12)
    rep = O.OFFSETS + O.OFFSETS[:3]
    np.testing.assert_array_equal(O.score_factored(k_post, p_q, centre, absmean, R, om, rep, "max"), mx)


# ---------------------------------------------------------------- decode loop
def _select_protected_bruteforce(scores, budget, sink, recent):
    """Every b-subset that holds all protected keys and in which each kept
    unprotected key beats each dropped key (same ranking as the top-B)."""
    s = np.asarray(scores, dtype=np.float64)
    n = len(s)
    b = min(budget, n)
    prot = {i for i in range(n) if i < sink or i >= n - recent}

    def beats(i, j):
        if np.isnan(s[i]) and np.isnan(s[j]):
            return i < j
        if np.isnan(s[i]):
            return False
        if np.isnan(s[j]):
            return True
        return s[i] > s[j] or (s[i] == s[j] and i < j)

    found = []
    for sub in itertools.combinations(range(n), b):
        kept = set(sub)
        if not prot <= kept:
            continue
        free_kept = kept - prot
        dropped = set(range(n)) - kept
        if all(beats(i, j) for i in free_kept for j in dropped):
            found.append(np.array(sub))
    assert len(found) == 1
    return found[0]


def test_select_protected_matches_enumeration():
    g = np.random.default_rng(21)
    pool = np.array([0.0, -0.0, 1.0, 1.0, -2.0, np.inf, -np.inf, np.nan, 3.5])
    for _ in range(300):
        n = int(g.integers(1, 9))
        sink = int(g.integers(0, 3))
        recent = int(g.integers(0, 3))
        prot = len({i for i in range(n) if i < sink or i >= n - recent})
        budget = int(g.integers(prot, n + 2))
        sc = g.choice(pool, size=n)
        np.testing.assert_array_equal(O.select_protected(sc, budget, sink, recent),
                                      _select_protected_bruteforce(sc, budget, sink, recent))


def test_select_protected_reduces_to_topb_and_to_the_protected_set():
    g = np.random.default_rng(22)
    for _ in range(50):
        n = int(g.integers(5, 60))
        sc = g.normal(size=n)
        b = int(g.integers(0, n + 3))
        np.testing.assert_array_equal(O.select_protected(sc, b, 0, 0), O.select_topb(sc, b))
        sink, recent = 2, 3
        if n >= 6:
            kept = O.select_protected(sc, sink + recent, sink, recent)
            np.testing.assert_array_equal(kept, np.r_[0:sink, n - recent:n])
    with pytest.raises(ValueError):
        O.select_protected(np.zeros(10), 3, 2, 2)


def _tiny_unit(n, d=8, seed=0):
    g = np.random.default_rng(seed)
    return O.DecodeUnit(g.integers(0, 2 ** 16, size=(n, d)), g.integers(0, 2 ** 16, size=(n, d)),
                        np.arange(n) * 3)


def test_decode_loop_keeps_oldest_and_recent_when_older_scores_higher():
    """score = -position: the oldest keys win, so after every prune the cache
    holds the first B - r positions ever seen plus the r newest."""
    B, I, r = 12, 5, 3
    u = _tiny_unit(B)
    seen = list(u.pos)
    prunes = 0
    for step in range(23):
        p = int(u.pos[-1]) + 2
        seen.append(p)
        sc = O.decode_step(u, np.full(8, step), np.full(8, step), p, B, I, 0, r,
                           lambda unit: -unit.pos.astype(float))
        if sc is not None:
            prunes += 1
            assert len(u) == B
            np.testing.assert_array_equal(u.pos, np.r_[seen[:B - r], seen[-r:]])
    assert prunes == 23 // I


def test_decode_loop_invariants():
    """Random scores: length sawtooth, prune count, time order, sink keys
    kept forever, the newest `recent` kept at every prune, kept rows are
    rows that were in the cache."""
    B, I, sink, recent = 20, 7, 2, 4
    u = _tiny_unit(B + 3, seed=5)
    g = np.random.default_rng(6)
    first = u.pos[:sink].copy()
    prunes = 0
    # prefill longer than B + I - 1 prunes at once in the driver; here the
    # unit starts below B + I
    for step in range(60):
        before = {int(x) for x in u.pos}
        p = int(u.pos[-1]) + 1 + int(g.integers(0, 3))
        before.add(p)
        newest = sorted(before)[-recent:]
        sc = O.decode_step(u, g.integers(0, 2 ** 16, 8), g.integers(0, 2 ** 16, 8), p, B, I,
                           sink, recent, lambda unit: g.normal(size=len(unit)))
        assert np.all(np.diff(u.pos) > 0)
        np.testing.assert_array_equal(u.pos[:sink], first)
        if sc is not None:
            prunes += 1
            assert len(u) == B
            assert set(newest) <= {int(x) for x in u.pos}
            assert {int(x) for x in u.pos} <= before
        else:
            assert len(u) < B + I
    assert prunes == (60 + 3) // I


# ------------------------------------------------- reconstruction diagnostic
def test_pearson_textbook_values():
    assert O.pearson([1, 2, 3], [2, 4, 6]) == pytest.approx(1.0, abs=1e-15)
    assert O.pearson([1, 2, 3], [3, 2, 1]) == pytest.approx(-1.0, abs=1e-15)
    # dx = dy-permuted (-1.5, -.5, .5, 1.5): sxy = 4, sxx = syy = 5
    assert O.pearson([1, 2, 3, 4], [1, 3, 2, 4]) == pytest.approx(0.8, abs=1e-15)
    assert O.pearson([2, 2, 2], [1, 5, 3]) == 0.0
    g = np.random.default_rng(31)
    x, y = g.normal(size=500), g.normal(size=500)
    assert O.pearson(x, y) == pytest.approx(np.corrcoef(x, y)[0, 1], abs=1e-12)
    assert O.pearson(3 * x + 1, -2 * y + 7) == pytest.approx(-O.pearson(x, y), abs=1e-12)


def _diag_case(noise, seed=0, nq=40, nk=60, d=16):
    g = np.random.default_rng(seed)
    om = O.rope_omega(d, 1e4)
    v = g.normal(size=d) + 1.0                      # one pre-RoPE direction
    q_pre = v[None, :] + noise * g.normal(size=(nq, d))
    q_pos = g.integers(0, 5000, size=nq).astype(np.float64)
    k_pos = np.sort(g.choice(4000, size=nk, replace=False)).astype(np.float64)
    k_pre = g.normal(size=(nk, d)) + 0.5
    q_post = O.rope_rotate(q_pre, q_pos, om)
    k_post = O.rope_rotate(k_pre, k_pos, om)
    centre, _, _ = O.calibrate(q_post[:, None, :], q_pos, om)
    return q_post, q_pos, k_post, k_pos, centre[0], om


def test_reconstruction_is_exact_when_queries_sit_on_their_centre():
    """Every sample query the same pre-RoPE vector: the centre is that vector
    and S_trig(k, Delta) is the logit itself (talk page, logit decomposition),
    so the two arrays agree entry by entry and r = 1."""
    q_post, q_pos, k_post, k_pos, centre, om = _diag_case(0.0)
    direct, recon = O.trig_reconstruction(q_post, q_pos, k_post, k_pos, centre, om)
    np.testing.assert_allclose(recon, direct, rtol=1e-11, atol=1e-11)
    assert O.trig_reconstruction_r(q_post, q_pos, k_post, k_pos, centre, om) == pytest.approx(1.0, abs=1e-12)


def test_reconstruction_degrades_with_query_spread():
    """Controlled concentration: the more the sample queries scatter around
    their centre, the lower the correlation (fixed seeds)."""
    rs = [O.trig_reconstruction_r(*_diag_case(noise, seed=4)) for noise in (0.02, 0.3, 1.0, 4.0)]
    assert rs[0] > 0.99
    assert all(a > b for a, b in zip(rs, rs[1:])), rs
    assert rs[-1] < 0.6


# ------------------------------------------------------------ per-layer budgets
def test_pyramid_budgets():
    b = O.pyramid_budgets(28, 2048, 3.0)
    assert len(b) == 28 and np.all(np.diff(b) >= 0)
    assert b[0] == 1024 and b[-1] == 3072                  # 2*2048/(1+3) and 3x that
    assert abs(b.mean() - 2048) <= 0.5
    np.testing.assert_array_equal(O.pyramid_budgets(5, 100, 1.0), [100] * 5)
    np.testing.assert_array_equal(O.pyramid_budgets(1, 77.5, 4.0), [78])
    np.testing.assert_array_equal(O.pyramid_budgets(3, 10, 3.0), [5, 10, 15])


def test_out_rows_layers_by_hand():
    """Two sequences of 5 and 3 keys, two layers, two KV heads; budgets
    [[2, 4], [9, 0]] keep (2, 4) and (3, 0) keys per unit."""
    cu, bud = [0, 5, 8], [[2, 4], [9, 0]]
    want = {(0, 0, 0): (0, 2), (0, 0, 1): (2, 2), (0, 1, 0): (4, 4), (0, 1, 1): (8, 4),
            (1, 0, 0): (12, 3), (1, 0, 1): (15, 3), (1, 1, 0): (18, 0), (1, 1, 1): (18, 0)}
    for key, val in want.items():
        assert O.out_rows_layers(cu, bud, 2, 2, *key) == val
    # with one budget per sequence it is the packed output layout
    for s in range(2):
        for l in range(2):
            for g in range(2):
                assert O.out_rows_layers(cu, [[3, 3], [2, 2]], 2, 2, s, l, g) == \
                    O.out_rows(cu, [3, 2], 2, 2, s, l, g)


# --------------------------------------------------------------------------
# Half-split RoPE layout (band f = x_f + i x_{f+d/2})
# --------------------------------------------------------------------------
def _to_half(x):
    """Column permutation interleaved -> half split: (x0, x2, .., x1, x3, ..)."""
    x = np.asarray(x)
    return np.concatenate([x[..., 0::2], x[..., 1::2]], axis=-1)


def test_half_split_quarter_turn_by_hand():
    g = GOLD["rope_quarter_turn_half_split"]
    om = O.rope_omega(g["d"], g["theta"])
    x = np.array(g["input"])
    np.testing.assert_allclose(O.rope_rotate(x, g["pos"], om, layout="half"), g["half"], atol=1e-15)
    np.testing.assert_allclose(O.rope_rotate(x, g["pos"], om), g["interleaved"], atol=1e-15)


def test_half_split_matches_rotate_half_form():
    """The usual half-split formula, x cos + rotate_half(x) sin with the
    angles repeated over both halves and rotate_half(x) = (-x2, x1)."""
    rng = np.random.default_rng(21)
    d = 64
    om = O.rope_omega(d, 1e4)
    x = rng.normal(size=(6, d))
    pos = rng.integers(0, 40000, size=6).astype(np.float64)
    ang = pos[:, None] * np.concatenate([om, om])[None, :]
    rot_half = np.concatenate([-x[:, d // 2:], x[:, :d // 2]], axis=1)
    want = x * np.cos(ang) + rot_half * np.sin(ang)
    np.testing.assert_allclose(O.rope_rotate(x, pos[:, None][:, 0], om, layout="half"), want,
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.rope_derotate(want, pos, om, layout="half"), x, atol=1e-12)


def test_half_split_relative_position_and_decomposition():
    rng = np.random.default_rng(22)
    d = 32
    om = O.rope_omega(d, 1e4)
    q, k = rng.normal(size=d), rng.normal(size=d)
    p1, p2 = 5000.0, 1234.0
    a = O.rope_rotate(q, p1, om, layout="half") @ O.rope_rotate(k, p2, om, layout="half")
    b = O.rope_rotate(q, p1 + 777, om, layout="half") @ O.rope_rotate(k, p2 + 777, om, layout="half")
    np.testing.assert_allclose(a, b, rtol=1e-10)
    np.testing.assert_allclose(O.logit_decomposed(q, k, p1 - p2, om, layout="half"), a, rtol=1e-10)


@pytest.mark.parametrize("reduce", ["mean", "max"])
@pytest.mark.parametrize("factored", [False, True])
def test_half_split_scores_equal_permuted_interleaved(reduce, factored):
    """Storing every vector with its columns permuted to the half layout and
    scoring with layout="half" reproduces the interleaved scores."""
    rng = np.random.default_rng(23)
    d, G, n = 32, 3, 40
    om = O.rope_omega(d, 1e4)
    k = rng.normal(size=(n, d))
    pos = np.sort(rng.choice(10000, size=n, replace=False)).astype(np.float64)
    centre = rng.normal(size=(G, d // 2)) + 1j * rng.normal(size=(G, d // 2))
    absmean = np.abs(centre) * 1.3
    R = np.abs(centre) / absmean
    offs = O.OFFSETS if reduce == "mean" else (1.0, 8.0, 100.0)
    a = O.unit_scores(k, pos, 12000.0, centre, absmean, R, om, offs, factored=factored,
                      reduce=reduce)
    b = O.unit_scores(_to_half(k), pos, 12000.0, centre, absmean, R, om, offs,
                      factored=factored, reduce=reduce, layout="half")
    np.testing.assert_allclose(b[0], a[0], atol=1e-9)
    np.testing.assert_allclose(b[1], a[1], rtol=1e-10, atol=1e-9)
    # planted mistake: reading half-split keys as interleaved changes them
    c = O.unit_scores(_to_half(k), pos, 12000.0, centre, absmean, R, om, offs,
                      factored=factored, reduce=reduce)
    assert np.max(np.abs(c[1] - a[1])) > 1e-3


def test_half_split_calibration_and_reconstruction():
    rng = np.random.default_rng(24)
    d, N, H = 16, 50, 2
    om = O.rope_omega(d, 1e4)
    q = rng.normal(size=(N, H, d)) + 2.0
    qpos = rng.integers(0, 5000, size=N)
    c1 = O.calibrate(q, qpos, om)
    c2 = O.calibrate(_to_half(q), qpos, om, layout="half")
    for x, y in zip(c1, c2):
        np.testing.assert_allclose(y, x, rtol=1e-12, atol=1e-12)
    k = rng.normal(size=(30, d))
    kpos = rng.integers(0, 5000, size=30)
    r1 = O.trig_reconstruction_r(q[:, 0], qpos, k, kpos, c1[0][0], om)
    r2 = O.trig_reconstruction_r(_to_half(q[:, 0]), qpos, _to_half(k), kpos, c1[0][0], om,
                                 layout="half")
    assert abs(r1 - r2) < 1e-12


# --------------------------------------------------------------------------
# Paged cache addressing
# --------------------------------------------------------------------------
def test_paged_rows_by_hand():
    g = GOLD["paged_rows_token_major"]
    P, H = g["P"], g["Hkv"]
    strides = (P * H, H, 1, 0)
    for s, l, h, i, row in g["cases"]:
        assert O.paged_row(g["table"], P, strides, s, l, h, i) == row


def test_paged_rows_reduce_to_packed_layout():
    """One sequence in one page whose strides are those of the packed layout
    (unit (l, g) holds n consecutive rows): the same rows as unit_rows."""
    n, L, H = 48, 3, 2
    strides = (0, 1, n, H * n)           # page, token, head, layer
    for l in range(L):
        for g in range(H):
            rows = O.paged_unit_rows([[0]], 64, strides, 0, l, g, n)
            start, nn = O.unit_rows([0, n], L, H, 0, l, g)
            np.testing.assert_array_equal(rows, np.arange(start, start + nn))


@pytest.mark.parametrize("head_major", [False, True])
def test_paged_rows_cover_the_pool_once(head_major):
    """Full pages under a permuted table: every pool row is used exactly once
    (token-major and head-major pages)."""
    rng = np.random.default_rng(31)
    P, L, H, S, pages_per_seq = 4, 2, 3, 3, 5
    npages = S * pages_per_seq
    table = rng.permutation(npages).reshape(S, pages_per_seq)
    page_rows = P * H
    strides = (page_rows, 1, P, npages * page_rows) if head_major else \
        (page_rows, H, 1, npages * page_rows)
    rows = np.concatenate([O.paged_unit_rows(table, P, strides, s, l, g, P * pages_per_seq)
                           for s in range(S) for l in range(L) for g in range(H)])
    np.testing.assert_array_equal(np.sort(rows), np.arange(L * npages * page_rows))
