"""tri_trig_correlation (reconstruction diagnostic) against the oracle.

Both sides get the same fp32 query centres (the oracle's calibration of the
sample queries, rounded to fp32) and the same bf16 queries and keys.  r is
a ratio of fp64 sums of fp32-accurate products: |r_gpu - r_ref| <= 2e-5.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import half_split
from synth.cases import _calibration_queries

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(shape, n_q, n_k, R_Q, seed, layout="interleaved"):
    import rope_aware_key_amd as R
    q, q_pos = _calibration_queries(shape, n_q, DEV, seed, R_Q=R_Q)
    case = synth.build_case("diag", shape, (n_k,), (1,), device=DEV, seed=seed, with_values=False)
    if layout == "half":
        d = shape.head_dim
        perm = torch.as_tensor(np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)]),
                               device=DEV)
        q = q[..., perm].contiguous()
        case = half_split(case)
    L, Hq, Hkv, d = shape.num_layers, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    om = O.rope_omega(d, shape.rope_theta)
    qb = O.bf16_bits_to_f64(q.cpu().numpy().view(np.uint16))           # [L, n_q, Hq, d]
    qp = q_pos.cpu().numpy().astype(np.float64)
    centre = np.zeros((L, Hq, d // 2, 2), np.float32)
    for l in range(L):
        c, _, _ = O.calibrate(qb[l], qp, om, layout=layout)
        centre[l, ..., 0], centre[l, ..., 1] = c.real, c.imag
    qc = torch.as_tensor(centre, device=DEV)
    sh = R.make_shape(d, Hq, Hkv, L, shape.rope_theta, rope_layout=layout)
    ws = torch.empty(R.tri_trig_correlation_workspace_bytes(sh, n_q), dtype=torch.uint8, device=DEV)
    r = torch.full((L, Hq), float("nan"), dtype=torch.float64, device=DEV)
    R.tri_trig_correlation(sh, q, q_pos, n_q, case.k, case.k_pos, n_k, qc, r, workspace=ws)
    torch.cuda.synchronize()
    r = r.cpu().numpy()
    kb = O.bf16_bits_to_f64(case.k.cpu().numpy().view(np.uint16))
    kp = case.k_pos.cpu().numpy().astype(np.float64)
    G = shape.group
    ref = np.zeros((L, Hq))
    for l in range(L):
        for h in range(Hq):
            u = l * Hkv + h // G
            c = centre[l, h, :, 0].astype(np.float64) + 1j * centre[l, h, :, 1].astype(np.float64)
            ref[l, h] = O.trig_reconstruction_r(qb[l, :, h, :], qp, kb[u * n_k:(u + 1) * n_k],
                                                kp[u * n_k:(u + 1) * n_k], c, om, layout=layout)
    return r, ref


@pytest.mark.parametrize("R_Q", [0.99, 0.8, 0.5])
def test_trig_correlation_matches_oracle(R_Q):
    """d = 128, G = 4, two layers; 100 queries and 300 keys (ragged tiles)."""
    shape = synth.Shape(128, 8, 2, 2)
    r, ref = _run(shape, 100, 300, R_Q, seed=int(R_Q * 100))
    np.testing.assert_allclose(r, ref, rtol=0, atol=2e-5)


@pytest.mark.parametrize("d,G,n_q,n_k", [(64, 2, 17, 33), (256, 1, 64, 64), (32, 8, 130, 15)])
def test_trig_correlation_shapes(d, G, n_q, n_k):
    shape = synth.Shape(d, 2 * G, 2, 1)
    r, ref = _run(shape, n_q, n_k, 0.9, seed=d)
    np.testing.assert_allclose(r, ref, rtol=0, atol=2e-5)


def test_trig_correlation_tracks_concentration():
    """Tighter query concentration, better reconstruction (per head)."""
    shape = synth.Shape(128, 4, 1, 1)
    hi, _ = _run(shape, 200, 500, 0.98, seed=1)
    lo, _ = _run(shape, 200, 500, 0.6, seed=1)
    assert np.all(hi > lo)
    assert np.all(hi > 0.9)


@pytest.mark.parametrize("seed", range(12))
def test_trig_correlation_random(seed):
    """Seeded random shapes (head_dim a multiple of 32 up to 256, group 1 to
    8, one or two layers, ragged query and key counts, either RoPE layout)."""
    g = np.random.default_rng([93, seed])
    d = int(g.integers(1, 9)) * 32
    G, Hkv, L = int(g.integers(1, 9)), int(g.integers(1, 3)), int(g.integers(1, 3))
    n_q, n_k = int(g.integers(1, 90)), int(g.integers(1, 200))
    layout = "half" if g.random() < 0.5 else "interleaved"
    shape = synth.Shape(d, G * Hkv, Hkv, L)
    r, ref = _run(shape, n_q, n_k, float(g.uniform(0.5, 0.99)), seed=100 + seed, layout=layout)
    np.testing.assert_allclose(r, ref, rtol=0, atol=2e-5)



@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 20) + 16 * 37, 64 << 20])
def test_stream_probe_reads_every_word(nbytes):
    """The read probe folds every 32-bit word of the buffer into the sink:
    its XOR equals the host's over the same bytes, for sizes that end in a
    partial grid stride."""
    import rope_aware_key_amd as R
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.as_tensor(words.view(np.int32), device=DEV)
    sink = torch.tensor([0x1234567], dtype=torch.int32, device=DEV)
    R.tri_stream_probe(src, sink)
    torch.cuda.synchronize()
    expect = np.bitwise_xor.reduce(words) ^ np.uint32(0x1234567)
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == expect
