"""Numerical bars of the parity tests (no torch: the oracle worker
processes use them too).

Scores are z-scores: |gpu - ref| <= 1e-4 * max(1, |ref|), floored at the
resolution fp32 raw scores allow (z_floor).  The floor is counted: every
unit compared notes its floor, and the session prints how many needed one
above 1e-4."""
import numpy as np

# units compared / units whose floor exceeded the plain 1e-4 bar / largest floor
FLOOR_STATS = {"units": 0, "above": 0, "max": 0.0}


def note_floor(floor: float):
    FLOOR_STATS["units"] += 1
    if floor > 1e-4:
        FLOOR_STATS["above"] += 1
    FLOOR_STATS["max"] = max(FLOOR_STATS["max"], float(floor))


def z_floor(S_ref: np.ndarray, sigma_ref: np.ndarray) -> float:
    """Resolution of a z-score computed from fp32 raw scores: the raw values
    carry a few ulps of |S~|, so z = (S~ - mu) / sigma carries about
    eps * |S~| / sigma.  64 ulps (2^-18) of the unit's largest |S~_h| / sigma_h;
    0 for a head with sigma = 0 (its z is 0 on both sides)."""
    ratios = [np.max(np.abs(S_ref[h])) / sigma_ref[h] for h in range(len(sigma_ref))
              if sigma_ref[h] > 0 and S_ref.shape[1] > 0]
    return 2.0 ** -18 * max(ratios) if ratios else 0.0


def score_error(gpu_scores: np.ndarray, ref: np.ndarray, floor=0.0) -> float:
    """Worst error on the 1e-4 scale: <= 1e-4 passes."""
    err = np.abs(gpu_scores.astype(np.float64) - ref) / np.maximum(1.0, np.abs(ref))
    bar = np.maximum(1e-4, floor / np.maximum(1.0, np.abs(ref)))
    return float(np.max(err / bar)) * 1e-4 if err.size else 0.0


def check_scores(gpu_scores: np.ndarray, ref: np.ndarray, what="", floor=0.0):
    """|gpu - ref| <= max(1e-4 * max(1, |ref|), floor): z-scores are in units
    of sigma; floor (z_floor) covers units whose spread is below the fp32
    resolution of their raw scores."""
    note_floor(floor)
    worst = score_error(gpu_scores, ref, floor)
    assert worst <= 1e-4, f"{what}: worst scaled score error {worst:.3e} (of the 1e-4 bar)"
    return worst


def check_raw(gpu_raw: np.ndarray, S_ref: np.ndarray, sigma_ref: np.ndarray, what=""):
    """Raw S~_h(i): |gpu - ref| <= 1e-4 * max(|ref|, sigma_h)."""
    scale = np.maximum(np.abs(S_ref), sigma_ref[:, None])
    err = np.abs(gpu_raw.T.astype(np.float64) - S_ref) / scale
    worst = float(np.max(err)) if err.size else 0.0
    assert worst <= 1e-4, f"{what}: worst scaled raw error {worst:.3e}"
    return worst


def head_stat_errors(hs_unit: np.ndarray, mu: np.ndarray, sigma: np.ndarray, S: np.ndarray):
    """(mu, sigma) of one unit against the oracle, as multiples of their bars
    (<= 1 passes): |mu_gpu - mu| <= 1e-5 * max(max sigma, max |S~|) and
    |sigma_gpu - sigma| <= 1e-5 * sigma + 1e-5 * max |S~|."""
    big = max(np.max(sigma), np.max(np.abs(S))) if S.size else 0.0
    amax = np.max(np.abs(S)) if S.size else 0.0
    e_mu = np.max(np.abs(hs_unit[:, 0] - mu)) / max(1e-5 * big, 1e-300)
    e_sig = np.max(np.abs(hs_unit[:, 1] - sigma) / np.maximum(1e-5 * sigma + 1e-5 * amax, 1e-300))
    return float(e_mu), float(e_sig)
