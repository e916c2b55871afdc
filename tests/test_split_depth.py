"""Why both MFMA score paths split each fp64 trig coefficient into two bf16
terms (hi + mid): in fp64, the z-scores computed with coefficients rounded
to two bf16 terms stay within 3e-5 (the averaged score, over units of the
five workload kinds) and 5e-5 (the maximum over the default offset set) of
the exact ones, well inside the 1e-4 score bar, while three terms stay
below 1e-7.  A split error of at most 2^-17 per coefficient moves a raw
score by a few 2^-17 of the raw scores' own spread.
"""
import numpy as np
import pytest

import oracle as O
import synth
from harness import unit_inputs


def _bf16(x):
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _split(x, terms):
    out, r = np.zeros_like(x), x.copy()
    for _ in range(terms):
        t = _bf16(r)
        out += t
        r = r - t
    return out


@pytest.mark.parametrize("shape,n,seed", [(synth.Shape(128, 7, 1, 1), 4096, 1),
                                          (synth.Shape(128, 4, 1, 1), 3200, 2),
                                          (synth.Shape(64, 8, 1, 1), 4096, 3)])
def test_two_bf16_terms_suffice_for_the_max_over_offsets(shape, n, seed):
    case = synth.build_case("split", shape, [n], [n // 8], seed=seed)
    d, G = shape.head_dim, shape.group
    om = O.rope_omega(d, shape.rope_theta)
    offs = np.array([2.0 ** j for j in range(17)])
    _, _, kbits, _, centre, absmean, Rr = unit_inputs(case, 0, 0, 0)
    kp = O.bf16_bits_to_f64(kbits)
    pq = float(case.cur_pos[0])
    A = centre[:, None, :] * np.exp(1j * om[None, None, :] * (pq + offs[None, :, None]))
    a = np.zeros((G, len(offs), d))
    a[..., 0::2], a[..., 1::2] = A.real, A.imag
    norm = np.abs(kp[:, 0::2] + 1j * kp[:, 1::2]) @ ((1 - Rr) * absmean).T

    def raw(coef):
        return (kp @ coef.reshape(-1, d).T).reshape(n, G, len(offs)).max(axis=2) + norm

    exact = raw(a)
    sigma = exact.std(axis=0)
    dz2 = np.max(np.abs(raw(_split(a, 2)) - exact) / sigma)
    dz3 = np.max(np.abs(raw(_split(a, 3)) - exact) / sigma)
    assert dz2 < 5e-5, dz2
    assert dz3 < 1e-7, dz3


@pytest.mark.parametrize("name,over,units", [
    ("decode_window", dict(S=2, L=2), 8),
    ("long_reasoning", dict(S=1, L=2, n=8192), 8),
    ("ragged", dict(S=4, L=1), 6),
    ("stress_ties", dict(n=16384), 4),
])
def test_two_bf16_terms_suffice_for_the_averaged_score(name, over, units):
    # the averaged score's coefficients a_h = E[q_f] C_f exp(i omega_f p_q),
    # C_f the mean of exp(i omega_f delta) over the default offsets
    case = synth.workload_case(name, **over)
    shape = case.shape
    d, G = shape.head_dim, shape.group
    om = O.rope_omega(d, shape.rope_theta)
    offs = np.array([2.0 ** j for j in range(17)])
    C = np.exp(1j * om[None, :] * offs[:, None]).mean(axis=0)
    worst2 = worst3 = 0.0
    done = 0
    for s in range(case.num_seqs):
        for l in range(shape.num_layers):
            for g in range(shape.num_kv_heads):
                if done == units:
                    break
                done += 1
                _, _, kbits, _, centre, absmean, Rr = unit_inputs(case, s, l, g)
                kp = O.bf16_bits_to_f64(kbits)
                A = centre * C[None, :] * np.exp(1j * om[None, :] * float(case.cur_pos[s]))
                a = np.zeros((G, d))
                a[:, 0::2], a[:, 1::2] = A.real, A.imag
                norm = np.abs(kp[:, 0::2] + 1j * kp[:, 1::2]) @ ((1 - Rr) * absmean).T
                exact = kp @ a.T + norm
                sigma = exact.std(axis=0)
                worst2 = max(worst2, np.max(np.abs(kp @ _split(a, 2).T + norm - exact) / sigma))
                worst3 = max(worst3, np.max(np.abs(kp @ _split(a, 3).T + norm - exact) / sigma))
    assert done == units
    assert worst2 < 3e-5, worst2
    assert worst3 < 1e-7, worst3
