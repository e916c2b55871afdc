"""Why the max-over-offsets path splits each trig coefficient into two
bf16 terms (hi + mid) while the averaged path keeps three: in fp64, the
z-scores of the maximum over the default offset set computed with
coefficients rounded to two bf16 terms stay within 5e-5 of the exact ones
(half the 1e-4 score bar) on synthetic units of the workloads' kind, and
three terms stay below 1e-7.  A split error of at most 2^-17 per
coefficient moves a raw score by a few 2^-17 of the raw scores' own spread.
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
