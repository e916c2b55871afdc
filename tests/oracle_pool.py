"""The factored fp64 oracle over many units in worker processes (test
infrastructure; imports no torch and touches no GPU).

The parent writes a case's arrays and the GPU's results to files that every
worker maps read-only (attach); each task scores a batch of units with the
oracle and returns, per unit, the error figures the parity bars use.  The
parent asserts on them, so a failure names its unit."""
import os

import numpy as np

import oracle as O
from checks import head_stat_errors, score_error, z_floor

_A = {}
_META = {}


def attach(files, meta):
    """Worker initializer: map the shared arrays; one BLAS thread per worker."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass
    for name, (path, dtype, shape) in files.items():
        _A[name] = np.memmap(path, dtype=np.dtype(dtype), mode="r", shape=tuple(shape))
    _META.update(meta)


def score_units(tasks):
    """tasks: [(u, s, l, g, start, n)].  Returns [(u, score_err, floor, mu_err,
    sigma_err)] with score_err on the 1e-4 scale and the head-stat errors as
    multiples of their bars."""
    G, d = _META["G"], _META["d"]
    om = O.rope_omega(d, _META["theta"])
    out = []
    for (u, s, l, g, start, n) in tasks:
        if n == 0:
            out.append((u, 0.0, 0.0, 0.0, 0.0))
            continue
        kbits = np.asarray(_A["k"][start:start + n])
        pos = np.asarray(_A["k_pos"][start:start + n]).astype(np.float64)
        hq = slice(g * G, (g + 1) * G)
        qc = np.asarray(_A["q_centre"][l, hq]).astype(np.float64)
        centre = qc[..., 0] + 1j * qc[..., 1]
        absmean = np.asarray(_A["q_absmean"][l, hq]).astype(np.float64)
        Rr = np.asarray(_A["q_R"][l, hq]).astype(np.float64)
        ref, S, mu, sigma = O.unit_scores(O.bf16_bits_to_f64(kbits), pos,
                                          float(_A["cur_pos"][s]), centre, absmean, Rr, om,
                                          factored=True, layout=_META["layout"])
        floor = z_floor(S, sigma)
        err = score_error(np.asarray(_A["scores"][start:start + n]), ref, floor)
        e_mu, e_sig = head_stat_errors(np.asarray(_A["head_stats"][u]), mu, sigma, S)
        out.append((u, err, floor, e_mu, e_sig))
    return out


def workers():
    """Worker processes: the host cores this process may use, at most 16 (one
    GPU's share of the host's cores on a shared machine)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))
