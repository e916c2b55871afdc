"""TriAttention KV-pruning oracle: a plain, slow, fp64 CPU implementation.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP library and imports nothing from it.

Sources (cited by page title and the section or equation on that page):

* [RoPE-eq]   qingkeai.online, talk page "聊聊 TriAttention: 面向长上下文推理的
              三角级数式 KV Cache 压缩" -- the RoPE rotation equation (band f,
              frequency omega_f = theta^(-2f/d), theta = 10000, 2x2 rotation).
* [logit-eq]  same page -- "RoPE 注意力 logit 的一般形式": logit(q,k) =
              sum_f |q_f||k_f| cos(omega_f*Delta + phi_f), Delta = p_q - p_k.
* [Strig-eq]  same page -- "三角级数分数" S_trig equation.
* [Snorm-eq]  same page -- "范数分数" S_norm equation and the definition of R_f.
* [avg-eq]    same page -- "综合打分并跨未来偏移平均": S = S_trig + S_norm and the
              mean over the offset set D = {1, 2, 4, ..., 2^16}.
* [topB]      same page -- the closing step: rank keys by the averaged score
              and keep the top B.
* [gqa]       hyper.ai summary of arXiv 2604.04921, section "方法": average over
              future query positions, then for grouped-query attention the
              scores are normalised before they are aggregated: z-score per
              query head, max over the group.
* [calib]     hyper.ai summary, section "方法" (R = |E[q]| / E[|q|]) and the
              shibing624 blog review, section "具体操作分三步" step 1 (offline
              calibration on ~10K tokens, done once).
* [evict]     jaedaily.cn KV-cache compression tutorial, eviction step
              (top-k, then the kept indices sorted so the time order is
              preserved, then keys and values gathered).
* [stream]    same tutorial page, streaming-generation paragraph: each decode
              step appends the new token's K and V, eviction runs when the
              cache exceeds the budget, and the most recent r tokens are
              protected; its renormalisation paragraph keeps attention-sink
              tokens (e.g. [BOS]).
* [trigger]   hyper.ai summary, section "方法": scoring and pruning run once
              every 128 generated tokens.
* [budget]    same tutorial page, budget-setting step: a KV budget B per
              layer, and pyramid-shaped allocation across layers (PyramidKV):
              fewer keys for shallow layers, more for deep ones.
* [layout]    the pages print only the interleaved pairing (x_2f, x_2f+1)
              of the talk page's rotation equation.  Pairing element f with
              element f + d/2 ("half split") is a storage layout the pages
              give no formula for; it is supported as a reading, each pair
              rotating by the printed matrix.
* [paged]     same tutorial page, deployment paragraph: engines keep the KV
              cache in pages (PagedAttention in vLLM), each sequence's
              logical blocks mapped to physical pages by a table.
* [recon]     shibing624 blog review, Fig. 1(D) (the trig series built from
              the centres against the real attention logits) and Fig. 7
              (per-head Pearson correlation of that reconstruction).

Readings where the pages are silent or disagree (each is a choice):

* RoPE pairs are interleaved (x_{2f}, x_{2f+1}) as the rotation equation
  writes them; band f is the complex number x_{2f} + i x_{2f+1}, and the
  printed matrix multiplies it by exp(+i omega_f p).  layout="half" takes
  band f as x_f + i x_{f+d/2} instead [layout]; nothing else changes.
* phi_f in S_trig is arg E[q_f] - arg k_f with k_f the pre-RoPE key.
* The offsets are averaged (formula page) by default; the blog review's
  maximum over D is available as reduce="max" (a variant, not the default).
* (1 - R_f) weights S_norm only.
* R_f := 1 when E|q_f| = 0 (both terms of that band vanish anyway).
* z-score uses the population standard deviation over all n keys of the
  unit; sigma = 0 gives z = 0.  Query heads [gG, (g+1)G) belong to KV head g.
* Ties in the top-B are broken by the lower position (= lower index, since
  positions increase within a unit); -0.0 equals +0.0; NaN ranks below -inf.
* Reconstruction diagnostic: per (layer, query head), the Pearson
  correlation over every (sample query, key) pair of the direct post-RoPE
  logit q'.k' and S_trig(k, p_q - p_k) built from the query centre; 0 when
  either side is constant.
* Pyramid budgets: linear in the layer index, b_l = round(b_0 + (b_{L-1} -
  b_0) l / (L - 1)) with b_{L-1} = ratio * b_0 and mean (b_0 + b_{L-1}) / 2
  equal to the requested mean (the pages give the shape, not a formula).
* Paged cache: a page holds P consecutive tokens of a sequence for every
  layer and KV head; one table per sequence (shared by its layers and heads)
  gives the physical page of each logical page; row strides per page, token,
  head and layer place every (page, slot, layer, head) row in the pool, so
  both head-major and token-major pages are described.
* Decode loop: a unit is pruned to B when it reaches B + interval keys
  (interval 128), scored at the position of its newest key; the first
  `sink` and the last `recent` keys are kept whatever their score and count
  against B; the other B - sink - recent are the top of the remaining keys
  by the same ranking as the top-B.
"""

from __future__ import annotations

import itertools

import numpy as np

# D = {2^0, 2^1, ..., 2^16}  [avg-eq]
OFFSETS = tuple(float(2 ** m) for m in range(17))


# --------------------------------------------------------------------------
# bf16 decoding (exact)
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16) to fp64 exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# RoPE  [RoPE-eq]
# --------------------------------------------------------------------------
def rope_omega(d: int, theta: float) -> np.ndarray:
    """omega_f = theta^(-2f/d) for f = 0 .. d/2-1."""
    if d % 2:
        raise ValueError("head_dim must be even")
    f = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * f / d)


LAYOUTS = ("interleaved", "half")


def _pair_slices(d: int, layout: str):
    """Element positions of (real, imaginary) parts of every band."""
    if layout == "interleaved":
        return slice(0, d, 2), slice(1, d, 2)
    if layout == "half":
        return slice(0, d // 2), slice(d // 2, d)
    raise ValueError(layout)


def rope_rotate(x: np.ndarray, pos, omega: np.ndarray, layout="interleaved") -> np.ndarray:
    """Apply the printed 2x2 rotation to every band of x at position pos.

    x: [..., d] (pre-RoPE).  pos broadcasts against x[..., 0].
    (x'_a, x'_b) = [[cos, -sin], [sin, cos]] (x_a, x_b), angle omega_f * pos,
    with (a, b) = (2f, 2f+1) (interleaved) or (f, f + d/2) (half).
    """
    x = np.asarray(x, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * omega
    c, s = np.cos(ang), np.sin(ang)
    ra, rb = _pair_slices(x.shape[-1], layout)
    xe, xo = x[..., ra], x[..., rb]
    out = np.empty_like(x)
    out[..., ra] = c * xe - s * xo
    out[..., rb] = s * xe + c * xo
    return out


def rope_derotate(x: np.ndarray, pos, omega: np.ndarray, layout="interleaved") -> np.ndarray:
    """Inverse of rope_rotate (rotation by -omega_f * pos)."""
    return rope_rotate(x, -np.asarray(pos, dtype=np.float64), omega, layout)


def bands(x: np.ndarray, layout="interleaved") -> np.ndarray:
    """View band f of x as the complex number x_a + i x_b, (a, b) as in
    rope_rotate."""
    x = np.asarray(x, dtype=np.float64)
    ra, rb = _pair_slices(x.shape[-1], layout)
    return x[..., ra] + 1j * x[..., rb]


# --------------------------------------------------------------------------
# Logit decomposition  [logit-eq]
# --------------------------------------------------------------------------
def logit_decomposed(q_pre: np.ndarray, k_pre: np.ndarray, delta, omega,
                     layout="interleaved") -> np.ndarray:
    """sum_f |q_f| |k_f| cos(omega_f * Delta + phi_f), phi_f = arg q_f - arg k_f.

    q_pre, k_pre: [..., d] pre-RoPE vectors; delta = p_q - p_k.
    """
    qf, kf = bands(q_pre, layout), bands(k_pre, layout)
    phi = np.angle(qf) - np.angle(kf)
    ang = np.asarray(delta, dtype=np.float64)[..., None] * omega + phi
    return np.sum(np.abs(qf) * np.abs(kf) * np.cos(ang), axis=-1)


# --------------------------------------------------------------------------
# Calibration  [calib], [Snorm-eq]
# --------------------------------------------------------------------------
def calibrate(q: np.ndarray, q_pos, omega: np.ndarray, layout="interleaved"):
    """Per-band query statistics from sample queries of one layer.

    q: [N, H, d] fp64 sample queries, post-RoPE at q_pos[N]; pass
       q_pos=None when the samples are already pre-RoPE.
    Returns (centre [H, F] complex = E[q_f],
             absmean [H, F] = E[|q_f|],
             R [H, F] = |E[q_f]| / E[|q_f|], with R := 1 where E|q_f| = 0).
    """
    q = np.asarray(q, dtype=np.float64)
    if q_pos is not None:
        pos = np.asarray(q_pos, dtype=np.float64)[:, None]       # [N, 1]
        q = rope_derotate(q, pos, omega, layout)                  # pre-RoPE
    qf = bands(q, layout)                                         # [N, H, F]
    centre = qf.mean(axis=0)
    absmean = np.abs(qf).mean(axis=0)
    R = np.ones_like(absmean)
    nz = absmean > 0
    R[nz] = np.abs(centre[nz]) / absmean[nz]
    return centre, absmean, R


# --------------------------------------------------------------------------
# Scores, term by term  [Strig-eq], [Snorm-eq], [avg-eq]
# --------------------------------------------------------------------------
def score_terms(k_post: np.ndarray, k_pos, p_q: float,
                centre: np.ndarray, absmean: np.ndarray, R: np.ndarray,
                omega: np.ndarray, offsets=OFFSETS, reduce="mean", layout="interleaved"):
    """Offset-reduced TriAttention score of every key, for each query head.

    k_post: [n, d] post-RoPE keys (fp64); k_pos: [n] their positions.
    centre/absmean/R: [G, F] statistics of the G query heads that read
    this KV head.  reduce: "mean" (the formula page's average over D) or
    "max" (the blog review's maximum over D).  Returns
    (S_tilde [G, n], S_trig_reduced [G, n], S_norm [G, n]).

    The trig term is summed band by band and offset by offset exactly as the
    equations write it; nothing is factored.  S_norm does not depend on the
    offset, so either reduction of S_trig + S_norm leaves it unchanged.
    """
    k_pre = rope_derotate(k_post, np.asarray(k_pos, dtype=np.float64), omega, layout)
    kf = bands(k_pre, layout)                           # [n, F]
    k_abs = np.abs(kf)
    k_arg = np.angle(kf)
    delta = p_q - np.asarray(k_pos, dtype=np.float64)   # [n]

    G = centre.shape[0]
    n = k_post.shape[0]
    s_trig = np.zeros((G, n))
    s_norm = np.zeros((G, n))
    for h in range(G):
        amp_q = np.abs(centre[h])                       # |E[q_f]|  [F]
        phi = np.angle(centre[h])[None, :] - k_arg      # [n, F]
        per = []
        for dlt in offsets:                             # S_trig at Delta + delta
            ang = (delta[:, None] + dlt) * omega[None, :] + phi
            per.append(np.sum(amp_q[None, :] * k_abs * np.cos(ang), axis=1))
        if reduce == "mean":
            s_trig[h] = np.sum(per, axis=0) / len(offsets)
        elif reduce == "max":
            s_trig[h] = np.max(per, axis=0)
        else:
            raise ValueError(reduce)
        # S_norm(k) = sum_f (1 - R_f) E|q_f| |k_f|; independent of Delta,
        # so the offset mean leaves it unchanged.
        s_norm[h] = np.sum(((1.0 - R[h]) * absmean[h])[None, :] * k_abs, axis=1)
    return s_trig + s_norm, s_trig, s_norm


def offset_phasor_mean(omega: np.ndarray, offsets=OFFSETS) -> np.ndarray:
    """C_f = mean over delta in D of exp(i omega_f delta)."""
    d = np.asarray(offsets, dtype=np.float64)
    return np.exp(1j * omega[:, None] * d[None, :]).mean(axis=1)


def score_factored(k_post: np.ndarray, p_q: float,
                   centre: np.ndarray, absmean: np.ndarray, R: np.ndarray,
                   omega: np.ndarray, offsets=OFFSETS, reduce="mean",
                   layout="interleaved") -> np.ndarray:
    """The same S_tilde as score_terms, written as one dot product per head.

    Band f of a query at p_q + delta contributes
    Re(E[q_f] conj(k_f) exp(i omega_f (Delta + delta))); with the stored key
    k'_f = k_f exp(i omega_f p_k) the key position cancels and the offset mean
    folds into C_f:  S_trig = sum_f Re(E[q_f] C_f exp(i omega_f p_q) conj(k'_f)).
    Used to check that identity and to evaluate large units quickly.  With
    reduce="max" the offsets cannot be folded: the dot product is taken per
    offset (A_f = E[q_f] exp(i omega_f (p_q + delta))) and the maximum kept.
    Returns S_tilde [G, n].
    """
    kf = bands(k_post, layout)                                   # [n, F]
    if reduce == "mean":
        C = offset_phasor_mean(omega, offsets)                   # [F]
        A = centre * C[None, :] * np.exp(1j * omega * p_q)[None, :]  # [G, F]
        trig = np.real(A[:, None, :] * np.conj(kf)[None, :, :]).sum(axis=2)
    elif reduce == "max":
        trig = None
        for dlt in offsets:
            A = centre * np.exp(1j * omega * (p_q + dlt))[None, :]
            t = np.real(A[:, None, :] * np.conj(kf)[None, :, :]).sum(axis=2)
            trig = t if trig is None else np.maximum(trig, t)
    else:
        raise ValueError(reduce)
    w = (1.0 - R) * absmean                                      # [G, F]
    norm = w @ np.abs(kf).T
    return trig + norm


# --------------------------------------------------------------------------
# GQA: normalise, then aggregate  [gqa]
# --------------------------------------------------------------------------
def zscore_rows(S: np.ndarray):
    """Per row (query head): z = (S - mean) / population std; std 0 -> z 0.

    Two passes (mean, then mean squared deviation).  Returns (z, mu, sigma).
    """
    S = np.asarray(S, dtype=np.float64)
    mu = S.mean(axis=1)
    sigma = np.sqrt(((S - mu[:, None]) ** 2).mean(axis=1))
    z = np.zeros_like(S)
    ok = sigma > 0
    z[ok] = (S[ok] - mu[ok, None]) / sigma[ok, None]
    return z, mu, sigma


def gqa_max(z: np.ndarray) -> np.ndarray:
    """Max over the query heads of one GQA group: [G, n] -> [n]."""
    return np.max(z, axis=0)


def unit_scores(k_post, k_pos, p_q, centre, absmean, R, omega,
                offsets=OFFSETS, factored=False, reduce="mean", layout="interleaved"):
    """Final fp64 score of each key of one unit (one sequence/layer/KV head).

    Returns (score [n], S_tilde [G, n], mu [G], sigma [G]).
    """
    if factored:
        S = score_factored(k_post, p_q, centre, absmean, R, omega, offsets, reduce, layout)
    else:
        S = score_terms(k_post, k_pos, p_q, centre, absmean, R, omega, offsets, reduce,
                        layout)[0]
    z, mu, sigma = zscore_rows(S)
    return gqa_max(z), S, mu, sigma


# --------------------------------------------------------------------------
# Top-B selection and order-preserving compaction  [topB], [evict]
# --------------------------------------------------------------------------
def select_topb(scores: np.ndarray, budget: int) -> np.ndarray:
    """Kept indices of one unit, ascending.

    b = min(budget, n).  Keys are ranked by score, higher first; equal
    scores go to the lower index (lower position); -0.0 equals +0.0; NaN
    ranks below every number.  The first b of that ranking are kept and
    returned in ascending index order (the time order).
    """
    s = np.asarray(scores)
    n = s.shape[0]
    b = max(0, min(int(budget), n))
    if b == 0:
        return np.zeros(0, dtype=np.int64)
    s64 = s.astype(np.float64)
    nan = np.isnan(s64)
    neg = np.where(nan, 0.0, -s64)            # -0.0 and +0.0 compare equal
    idx = np.arange(n)
    order = np.lexsort((idx, neg, nan.astype(np.int8)))  # last key sorts first
    return np.sort(order[:b])


def select_topb_bruteforce(scores: np.ndarray, budget: int) -> np.ndarray:
    """Definition by enumeration (tiny n only): the unique b-subset S such
    that every kept key beats every dropped one, where i beats j if
    score_i > score_j, or the scores are equal and i < j (NaN below all,
    -0 == +0)."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    b = max(0, min(int(budget), n))

    def beats(i, j):
        si, sj = s[i], s[j]
        if np.isnan(si) and np.isnan(sj):
            return i < j
        if np.isnan(si):
            return False
        if np.isnan(sj):
            return True
        if si != sj:
            return si > sj
        return i < j

    found = []
    for sub in itertools.combinations(range(n), b):
        kept = set(sub)
        if all(beats(i, j) for i in kept for j in range(n) if j not in kept):
            found.append(np.array(sub, dtype=np.int64))
    if len(found) != 1:
        raise AssertionError(f"expected one valid subset, found {len(found)}")
    return found[0]


def compact_rows(rows: np.ndarray, kept: np.ndarray) -> np.ndarray:
    """Gather rows[kept] (keys, values or positions) in the given order."""
    return np.asarray(rows)[np.asarray(kept, dtype=np.int64)]


# --------------------------------------------------------------------------
# Whole-batch helpers over the unit-major packed layout
# --------------------------------------------------------------------------
def unit_rows(cu_len, L: int, Hkv: int, s: int, l: int, g: int):
    """Row range [start, start+n) of unit (s, l, g) in the packed cache:
    sequence s starts at L*Hkv*cu_len[s]; unit (l, g) holds n_s rows."""
    n = int(cu_len[s + 1] - cu_len[s])
    start = L * Hkv * int(cu_len[s]) + (l * Hkv + g) * n
    return start, n


def out_rows(cu_len, budget, L: int, Hkv: int, s: int, l: int, g: int):
    """Output row range of unit (s, l, g): as unit_rows with b_s = min(B_s, n_s)."""
    b = [max(0, min(int(budget[i]), int(cu_len[i + 1] - cu_len[i])))
         for i in range(len(cu_len) - 1)]
    cu_b = np.concatenate([[0], np.cumsum(b)]).astype(np.int64)
    start = L * Hkv * int(cu_b[s]) + (l * Hkv + g) * b[s]
    return start, b[s]


# --------------------------------------------------------------------------
# Decode loop: append, prune every `interval` tokens, keep sink and recent
# keys  [stream], [trigger]
# --------------------------------------------------------------------------
def protected_mask(n: int, sink: int, recent: int) -> np.ndarray:
    """Keys that are always kept: the first `sink` and the last `recent`."""
    i = np.arange(n)
    return (i < sink) | (i >= n - recent)


def select_protected(scores: np.ndarray, budget: int, sink: int, recent: int) -> np.ndarray:
    """Kept indices (ascending): every protected key, plus the top
    b - (#protected) of the other keys ranked as in select_topb, with
    b = min(budget, n) and #protected <= b."""
    s = np.asarray(scores)
    n = s.shape[0]
    b = max(0, min(int(budget), n))
    prot = protected_mask(n, sink, recent)
    n_prot = int(prot.sum())
    if n_prot > b:
        raise ValueError("more protected keys than the budget")
    free = np.nonzero(~prot)[0]
    chosen = free[select_topb(s[free], b - n_prot)]
    return np.sort(np.concatenate([np.nonzero(prot)[0], chosen]))


class DecodeUnit:
    """One (sequence, layer, KV head) cache in the decode loop: bf16 key and
    value rows (raw 16-bit patterns) and int positions, in time order."""

    def __init__(self, k_bits, v_bits, pos):
        """k_bits, v_bits: [n, d] raw bf16 patterns; pos: [n]."""
        self.k = np.asarray(k_bits, dtype=np.uint16)
        self.v = np.asarray(v_bits, dtype=np.uint16)
        self.pos = np.asarray(pos, dtype=np.int64)
        assert self.k.ndim == 2 and self.k.shape == self.v.shape and len(self.k) == len(self.pos)

    def __len__(self):
        return len(self.pos)

    def append(self, k_row, v_row, p):
        self.k = np.vstack([self.k, np.asarray(k_row, dtype=np.uint16)[None]])
        self.v = np.vstack([self.v, np.asarray(v_row, dtype=np.uint16)[None]])
        self.pos = np.append(self.pos, int(p))

    def scores(self, centre, absmean, R, omega, offsets=OFFSETS, reduce="mean",
               factored=False, p_q=None, layout="interleaved"):
        """Final scores of every key, the query at the newest key's position
        (or at p_q)."""
        p = float(self.pos[-1]) if p_q is None else float(p_q)
        return unit_scores(bf16_bits_to_f64(self.k), self.pos.astype(np.float64), p, centre,
                           absmean, R, omega, offsets, factored=factored, reduce=reduce,
                           layout=layout)[0]

    def prune(self, kept):
        kept = np.asarray(kept, dtype=np.int64)
        self.k, self.v, self.pos = (compact_rows(self.k, kept), compact_rows(self.v, kept),
                                    compact_rows(self.pos, kept))


def decode_step(unit: DecodeUnit, k_row, v_row, p, budget, interval, sink, recent,
                score_fn):
    """Append one token; if the unit now holds budget + interval keys, score
    it (score_fn(unit) -> scores) and keep select_protected of them.
    Returns the scores used, or None when no prune ran."""
    unit.append(k_row, v_row, p)
    if len(unit) < budget + interval:
        return None
    sc = score_fn(unit)
    unit.prune(select_protected(sc, budget, sink, recent))
    return sc


# --------------------------------------------------------------------------
# Reconstruction diagnostic  [recon], [logit-eq], [Strig-eq]
# --------------------------------------------------------------------------
def pearson(x, y) -> float:
    """Pearson correlation of two equal-length samples from centred fp64
    sums; 0 when either sample is constant."""
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    dx, dy = x - x.mean(), y - y.mean()
    sxx, syy = float(np.sum(dx * dx)), float(np.sum(dy * dy))
    if sxx == 0.0 or syy == 0.0:
        return 0.0
    return float(np.sum(dx * dy)) / np.sqrt(sxx * syy)


def trig_reconstruction(q_post, q_pos, k_post, k_pos, centre, omega, layout="interleaved"):
    """For one (layer, query head): the direct logits [n_q, n_k], q'_j . k'_i
    of the post-RoPE vectors, and the reconstruction S_trig(k_i, p_j - p_i)
    = sum_f |E q_f| |k_f| cos(omega_f Delta + arg E q_f - arg k_f) with k_f
    the pre-RoPE key band and E q_f = centre [F] complex."""
    q_post = np.asarray(q_post, dtype=np.float64)
    k_post = np.asarray(k_post, dtype=np.float64)
    direct = q_post @ k_post.T
    k_pre = rope_derotate(k_post, np.asarray(k_pos, dtype=np.float64), omega, layout)
    c_vec = np.empty(2 * len(centre))
    ra, rb = _pair_slices(len(c_vec), layout)
    c_vec[ra], c_vec[rb] = np.real(centre), np.imag(centre)
    delta = np.asarray(q_pos, dtype=np.float64)[:, None] - np.asarray(k_pos, dtype=np.float64)[None, :]
    recon = logit_decomposed(c_vec[None, None, :], k_pre[None, :, :], delta, omega, layout)
    return direct, recon


def trig_reconstruction_r(q_post, q_pos, k_post, k_pos, centre, omega,
                          layout="interleaved") -> float:
    """Pearson r of the reconstruction against the direct logits, over all
    (query, key) pairs."""
    direct, recon = trig_reconstruction(q_post, q_pos, k_post, k_pos, centre, omega, layout)
    return pearson(recon, direct)


# --------------------------------------------------------------------------
# Per-layer budgets  [budget]
# --------------------------------------------------------------------------
def pyramid_budgets(L: int, mean_budget: float, ratio: float) -> np.ndarray:
    """Budgets per layer growing linearly from the first layer to the last:
    the last is `ratio` times the first and the two ends average to
    mean_budget; each is rounded to the nearest integer (halves up)."""
    if L == 1:
        return np.array([int(np.floor(mean_budget + 0.5))])
    b0 = 2.0 * mean_budget / (1.0 + ratio)
    b1 = ratio * b0
    return np.floor(b0 + (b1 - b0) * np.arange(L) / (L - 1) + 0.5).astype(np.int64)


def out_rows_layers(cu_len, budgets, L: int, Hkv: int, s: int, l: int, g: int):
    """Output rows of unit (s, l, g) when each (sequence, layer) has its own
    budget budgets[s][l]: (sequence, layer) pairs in order, each holding its
    Hkv units of b = min(budgets[s][l], n_s) rows back to back."""
    acc = 0
    for s2 in range(len(cu_len) - 1):
        n = int(cu_len[s2 + 1] - cu_len[s2])
        for l2 in range(L):
            b = max(0, min(int(budgets[s2][l2]), n))
            if (s2, l2) == (s, l):
                return acc + g * b, b
            acc += Hkv * b
    raise IndexError((s, l, g))


# --------------------------------------------------------------------------
# Paged cache addressing  [paged]
# --------------------------------------------------------------------------
def paged_row(table, P: int, strides, s: int, l: int, g: int, i: int) -> int:
    """Pool row of token i of unit (s, l, g): logical page i // P of sequence
    s is physical page table[s][i // P], slot i % P within it.  strides =
    (page, token, head, layer) row strides."""
    page_st, token_st, head_st, layer_st = strides
    page = int(table[s][i // P])
    return l * layer_st + g * head_st + page * page_st + (i % P) * token_st


def paged_unit_rows(table, P: int, strides, s: int, l: int, g: int, n: int) -> np.ndarray:
    """Pool rows of the n tokens of unit (s, l, g), in token order."""
    return np.array([paged_row(table, P, strides, s, l, g, i) for i in range(n)], dtype=np.int64)

