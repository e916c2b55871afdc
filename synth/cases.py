"""Seeded synthetic inputs for the TriAttention pruning path.

This module only makes data: a post-RoPE bf16 key cache with concentrated
pre-RoPE keys, values, positions, per-band query statistics (or raw
calibration queries) and the per-sequence lengths, current positions and
budgets.  It contains none of the scoring, selection or compaction
arithmetic; both the HIP library's tests and the CPU oracle consume what it
returns.

Workload shapes follow the long-reasoning setting the pages evaluate
(32K-token generation, budgets 512-4096, ~10K calibration tokens, heads
whose pre-RoPE queries and keys sit close to a fixed centre with
concentration R mostly above 0.9 -- shibing624 blog review, sections
"核心发现" and "方法"; hyper.ai summary, section "方法").  No dataset or model
weight is used: the synthetic caches stand in for them.

Keys are built pre-RoPE as  k_f = c_f + rho(R_K) |c_f| (N(0,1) + i N(0,1))
per band (c_f = per (layer, KV head, band) centre with |c_f| ~ U[0.5, 2] and
uniform phase), then rotated to their positions with the RoPE of the
qingkeai.online talk page (band f multiplied by exp(+i omega_f p),
omega_f = theta^(-2f/d)), then rounded to bf16.  rho(R) is the noise ratio
for which a complex Gaussian around a centre has mean resultant length R
(Rice mean), found by bisection.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from functools import lru_cache
from typing import Optional

import numpy as np
import torch

SEED_BASE = 20260406


@dataclass(frozen=True)
class Shape:
    head_dim: int
    num_q_heads: int
    num_kv_heads: int
    num_layers: int
    rope_theta: float = 10000.0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def bands(self) -> int:
        return self.head_dim // 2


@dataclass
class Case:
    name: str
    shape: Shape
    cu_len: np.ndarray          # int64 [S+1], host
    cur_pos: np.ndarray         # int32 [S], host
    budget: np.ndarray          # int32 [S], host
    k: torch.Tensor             # int16 bf16 bits [rows, d] (post-RoPE)
    v: Optional[torch.Tensor]   # int16 bf16 bits [rows, d]
    k_pos: torch.Tensor         # int32 [rows]
    q_centre: torch.Tensor      # float32 [L, Hq, F, 2]
    q_absmean: torch.Tensor     # float32 [L, Hq, F]
    q_R: torch.Tensor           # float32 [L, Hq, F]
    calib_q: Optional[torch.Tensor] = None    # int16 bf16 bits [L, N, Hq, d]
    calib_pos: Optional[torch.Tensor] = None  # int32 [N]
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.cu_len) - 1

    @property
    def num_units(self) -> int:
        return self.num_seqs * self.shape.num_layers * self.shape.num_kv_heads

    def seq_len(self, s: int) -> int:
        return int(self.cu_len[s + 1] - self.cu_len[s])

    def kept(self, s: int) -> int:
        return max(0, min(int(self.budget[s]), self.seq_len(s)))

    def out_cu(self) -> np.ndarray:
        key = (np.asarray(self.budget).tobytes(), np.asarray(self.cu_len).tobytes())
        cached = self.meta.get("_out_cu")
        if cached is None or cached[0] != key:
            lens = np.diff(np.asarray(self.cu_len, dtype=np.int64))
            b = np.clip(np.minimum(np.asarray(self.budget, dtype=np.int64), lens), 0, None)
            cached = (key, np.concatenate([[0], np.cumsum(b)]).astype(np.int64))
            self.meta["_out_cu"] = cached
        return cached[1]

    def total_rows(self) -> int:
        return int(self.cu_len[-1]) * self.shape.num_layers * self.shape.num_kv_heads

    def total_out_rows(self) -> int:
        return int(self.out_cu()[-1]) * self.shape.num_layers * self.shape.num_kv_heads

    def unit_rows(self, s, l, g):
        n = self.seq_len(s)
        L, H = self.shape.num_layers, self.shape.num_kv_heads
        return L * H * int(self.cu_len[s]) + (l * H + g) * n, n

    def unit_out_rows(self, s, l, g):
        b = self.kept(s)
        L, H = self.shape.num_layers, self.shape.num_kv_heads
        return L * H * int(self.out_cu()[s]) + (l * H + g) * b, b


# ---------------------------------------------------------------------------
@lru_cache(maxsize=None)
def noise_ratio(R: float) -> float:
    """Per-component noise std / |centre| giving mean resultant length R."""
    from scipy.special import i0e, i1e

    def r_of(rho):
        x = -1.0 / (2.0 * rho * rho)
        y = -x / 2.0
        lag = (1.0 - x) * i0e(y) - x * i1e(y)
        return 1.0 / (rho * math.sqrt(math.pi / 2.0) * lag)

    lo, hi = 1e-4, 100.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if r_of(mid) > R:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _gen(device, *tags) -> torch.Generator:
    g = torch.Generator(device=device)
    h = SEED_BASE
    for t in tags:
        h = (h * 1000003 + int(t)) % (2 ** 61 - 1)
    g.manual_seed(h)
    return g


def _stable_tag(s: str) -> int:
    return sum((i + 1) * ord(c) for i, c in enumerate(s))


def _gen_t(device, *tags) -> torch.Generator:
    return _gen(device, *[_stable_tag(t) if isinstance(t, str) else t for t in tags])


def _to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).view(torch.int16)


def _rotate(re: torch.Tensor, im: torch.Tensor, pos: torch.Tensor, theta: float, d: int):
    """Post-RoPE interleaved rows from pre-RoPE band parts (model-side RoPE).

    re, im: [..., n, F] fp32; pos: [n] (int).  Angles in fp64."""
    F = d // 2
    f = torch.arange(F, device=re.device, dtype=torch.float64)
    om = torch.pow(torch.tensor(theta, dtype=torch.float64, device=re.device), -2.0 * f / d)
    ang = pos.to(torch.float64)[:, None] * om[None, :]
    c = torch.cos(ang).to(torch.float32)
    s = torch.sin(ang).to(torch.float32)
    out = torch.empty(re.shape[:-1] + (d,), dtype=torch.float32, device=re.device)
    out[..., 0::2] = c * re - s * im
    out[..., 1::2] = s * re + c * im
    return out


def _key_centres(shape: Shape, device, seed, tag="kcentre"):
    L, H, F = shape.num_layers, shape.num_kv_heads, shape.bands
    g = _gen_t(device, seed, tag)
    amp = torch.rand(L, H, F, generator=g, device=device) * 1.5 + 0.5
    ph = torch.rand(L, H, F, generator=g, device=device) * (2 * math.pi)
    return amp * torch.cos(ph), amp * torch.sin(ph)


def _query_stats(shape: Shape, device, seed, r_lo=0.6, r_hi=0.99, low_mask=None, low_R=0.3):
    """Per (layer, q head, band) statistics synthesised directly:
    R ~ U[r_lo, r_hi], |E q| ~ U[0.5, 2], arg E q ~ U[0, 2pi), E|q| = |E q| / R."""
    L, Hq, F = shape.num_layers, shape.num_q_heads, shape.bands
    g = _gen_t(device, seed, "qstats")
    R = torch.rand(L, Hq, F, generator=g, device=device) * (r_hi - r_lo) + r_lo
    if low_mask is not None:
        R = torch.where(low_mask, torch.full_like(R, low_R), R)
    amp = torch.rand(L, Hq, F, generator=g, device=device) * 1.5 + 0.5
    ph = torch.rand(L, Hq, F, generator=g, device=device) * (2 * math.pi)
    centre = torch.stack([amp * torch.cos(ph), amp * torch.sin(ph)], dim=-1)
    absmean = amp / R
    # store exactly what the fp32 arrays hold; R is recomputed by neither side
    return centre.float().contiguous(), absmean.float().contiguous(), R.float().contiguous()


def _fill_keys(case_shape: Shape, k: torch.Tensor, cu_len, positions, seed, device,
               rho_of_band=None, dup_blocks=False, chunk_rows=1 << 22):
    """Write post-RoPE bf16 keys for every unit into k (int16 view)."""
    L, H, d, F = case_shape.num_layers, case_shape.num_kv_heads, case_shape.head_dim, case_shape.bands
    cre, cim = _key_centres(case_shape, device, seed)
    rho_default = noise_ratio(0.95)
    S = len(cu_len) - 1
    for s in range(S):
        n = int(cu_len[s + 1] - cu_len[s])
        if n == 0:
            continue
        pos = positions[s]
        for l in range(L):
            g = _gen_t(device, seed, "keys", s, l)
            base = L * H * int(cu_len[s]) + l * H * n
            # H units of this (s, l) are contiguous: rows [base, base + H n)
            step = max(1, chunk_rows // max(1, n))
            for h0 in range(0, H, step):
                h1 = min(H, h0 + step)
                nh = h1 - h0
                rho = torch.full((nh, 1, F), rho_default, device=device)
                if rho_of_band is not None:
                    rho = rho_of_band[l, h0:h1][:, None, :].to(device)
                amp = torch.sqrt(cre[l, h0:h1] ** 2 + cim[l, h0:h1] ** 2)[:, None, :]
                nre = torch.randn(nh, n, F, generator=g, device=device)
                nim = torch.randn(nh, n, F, generator=g, device=device)
                re = cre[l, h0:h1][:, None, :] + rho * amp * nre
                im = cim[l, h0:h1][:, None, :] + rho * amp * nim
                rows = _to_bf16_bits(_rotate(re, im, pos, case_shape.rope_theta, d))
                if dup_blocks:
                    # post-RoPE duplicates: rows [128j+64, 128j+128) copy [128j, 128j+64)
                    j = torch.arange(n, device=device)
                    dst = j[(j % 128) >= 64]
                    rows[:, dst] = rows[:, dst - 64]
                k[base + h0 * n: base + h1 * n] = rows.reshape(nh * n, d)


def _fill_values(v: torch.Tensor, seed, device, chunk_rows=1 << 24):
    g = _gen_t(device, seed, "values")
    rows = v.shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        v[r0:r1] = _to_bf16_bits(torch.randn(r1 - r0, v.shape[1], generator=g, device=device))


def _fill_positions(k_pos: torch.Tensor, shape: Shape, cu_len, positions):
    L, H = shape.num_layers, shape.num_kv_heads
    for s in range(len(cu_len) - 1):
        n = int(cu_len[s + 1] - cu_len[s])
        if n == 0:
            continue
        base = L * H * int(cu_len[s])
        k_pos[base: base + L * H * n] = positions[s].to(torch.int32).repeat(L * H)


def _calibration_queries(shape: Shape, n_samples, device, seed, R_Q=0.95):
    """Synthetic post-RoPE bf16 queries at positions 0..N-1, concentrated
    around a separate per (layer, q head, band) centre."""
    L, Hq, d, F = shape.num_layers, shape.num_q_heads, shape.head_dim, shape.bands
    g = _gen_t(device, seed, "qcentre")
    amp = torch.rand(L, Hq, F, generator=g, device=device) * 1.5 + 0.5
    ph = torch.rand(L, Hq, F, generator=g, device=device) * (2 * math.pi)
    cre, cim = amp * torch.cos(ph), amp * torch.sin(ph)
    rho = noise_ratio(R_Q)
    pos = torch.arange(n_samples, device=device, dtype=torch.int64)
    out = torch.empty(L, n_samples, Hq, d, dtype=torch.int16, device=device)
    for l in range(L):
        gg = _gen_t(device, seed, "queries", l)
        nre = torch.randn(Hq, n_samples, F, generator=gg, device=device)
        nim = torch.randn(Hq, n_samples, F, generator=gg, device=device)
        re = cre[l][:, None, :] + rho * amp[l][:, None, :] * nre
        im = cim[l][:, None, :] + rho * amp[l][:, None, :] * nim
        rows = _rotate(re, im, pos, shape.rope_theta, d)       # [Hq, N, d]
        out[l] = _to_bf16_bits(rows.permute(1, 0, 2))
    return out.contiguous(), pos.to(torch.int32)


# ---------------------------------------------------------------------------
def build_case(name: str, shape: Shape, seq_lens, budgets, device="cpu", seed=0,
               positions=None, cur_pos=None, with_values=True, stats="synthetic",
               calib_samples=10240, low_band_frac=0.0, dup_blocks=False) -> Case:
    """Assemble a packed, unit-major case.

    seq_lens/budgets: per sequence.  positions: list of int64 tensors
    (default 0..n-1); cur_pos: per sequence (default n).
    stats: "synthetic" (statistics drawn directly) or "calibrate" (raw
    post-RoPE queries are produced; statistics are left zero for the
    caller to fill from a calibration run).
    """
    device = torch.device(device)
    S = len(seq_lens)
    cu_len = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int64)
    if positions is None:
        positions = [torch.arange(int(n), dtype=torch.int64, device=device) for n in seq_lens]
    if cur_pos is None:
        cur_pos = [int(p[-1].item()) + 1 if len(p) else 0 for p in positions]
    cur_pos = np.asarray(cur_pos, dtype=np.int32)
    budget = np.asarray(budgets, dtype=np.int32)
    L, H, d, F = shape.num_layers, shape.num_kv_heads, shape.head_dim, shape.bands
    rows = int(cu_len[-1]) * L * H

    low_mask_q = None
    rho_of_band = None
    if low_band_frac > 0:
        gm = _gen_t(device, seed, "lowbands")
        low_kv = torch.rand(L, H, F, generator=gm, device=device) < low_band_frac
        rho_of_band = torch.where(low_kv, torch.full(low_kv.shape, noise_ratio(0.3), device=device),
                                  torch.full(low_kv.shape, noise_ratio(0.95), device=device))
        low_mask_q = low_kv.repeat_interleave(shape.group, dim=1)

    k = torch.empty(rows, d, dtype=torch.int16, device=device)
    _fill_keys(shape, k, cu_len, positions, seed, device, rho_of_band=rho_of_band, dup_blocks=dup_blocks)
    v = None
    if with_values:
        v = torch.empty(rows, d, dtype=torch.int16, device=device)
        _fill_values(v, seed, device)
    k_pos = torch.empty(rows, dtype=torch.int32, device=device)
    _fill_positions(k_pos, shape, cu_len, positions)

    calib_q = calib_pos = None
    if stats == "calibrate":
        calib_q, calib_pos = _calibration_queries(shape, calib_samples, device, seed)
        Hq = shape.num_q_heads
        qc = torch.zeros(L, Hq, F, 2, device=device)
        qa = torch.zeros(L, Hq, F, device=device)
        qr = torch.zeros(L, Hq, F, device=device)
    else:
        qc, qa, qr = _query_stats(shape, device, seed, low_mask=low_mask_q)
    return Case(name, shape, cu_len, cur_pos, budget, k, v, k_pos, qc, qa, qr,
                calib_q, calib_pos, meta={"seed": seed})


# ---------------------------------------------------------------------------
# The five workloads, by name; keyword overrides shrink batch, layers or
# lengths for tests.
#   smallest         1 unit of 4096 keys -> 512, d 128, stats from calibration
#   decode_window    64 seq x 32 layers x 8 KV heads (G 4), 3200 keys -> 3072
#   long_reasoning   8 seq x 28 layers x 4 KV heads (G 7), 32768 keys -> 2048
#   ragged           256 seq of 2048..16384 keys, budgets 1024/2048/3072, G 4
#   stress_ties      d 64, G 8, 131072 keys -> 4096, weak bands, twin blocks
# ---------------------------------------------------------------------------
WORKLOAD_NAMES = ("smallest", "decode_window", "long_reasoning", "ragged", "stress_ties")


def workload_case(name: str, device="cpu", seed=0, **over) -> Case:
    if name == "smallest":
        shape = Shape(128, 1, 1, 1)
        return build_case("smallest_4096_to_512", shape, [over.get("n", 4096)],
                          [over.get("B", 512)], device=device, seed=seed, stats="calibrate",
                          calib_samples=over.get("calib_samples", 10240))
    if name == "decode_window":
        S = over.get("S", 64)
        L = over.get("L", 32)
        shape = Shape(128, 32, 8, L)
        n, B, win = over.get("n", 3200), over.get("B", 3072), 128
        g = np.random.default_rng([SEED_BASE, 2, seed])
        positions, cur = [], []
        for _ in range(S):
            pq = int(g.integers(8192, 32769))
            old = np.sort(g.choice(pq - win, size=n - win, replace=False))
            pos = np.concatenate([old, np.arange(pq - win, pq)])
            positions.append(torch.as_tensor(pos, dtype=torch.int64, device=device))
            cur.append(pq)
        return build_case("decode_window_3200_to_3072", shape, [n] * S, [B] * S, device=device,
                          seed=seed, positions=positions, cur_pos=cur)
    if name == "long_reasoning":
        S = over.get("S", 8)
        L = over.get("L", 28)
        n = over.get("n", 32768)
        shape = Shape(128, 28, 4, L)
        return build_case("long_reasoning_32k_to_2048", shape, [n] * S,
                          [over.get("B", 2048)] * S, device=device, seed=seed)
    if name == "ragged":
        S = over.get("S", 256)
        L = over.get("L", 1)
        lo, hi = over.get("n_range", (2048, 16384))
        shape = Shape(128, 32, 8, L)
        g = np.random.default_rng([SEED_BASE, 4, seed])
        lens = g.integers(lo, hi + 1, size=S).tolist()
        budgets = g.choice([1024, 2048, 3072], size=S).tolist()
        if "budgets" in over:
            budgets = over["budgets"]
        return build_case("ragged_256seq", shape, lens, budgets, device=device, seed=seed)
    if name == "stress_ties":
        n = over.get("n", 131072)
        S = over.get("S", 1)
        shape = Shape(64, 64, 8, over.get("L", 1))
        return build_case("stress_ties_131072_to_4096", shape, [n] * S, [over.get("B", 4096)] * S,
                          device=device, seed=seed, low_band_frac=0.1, dup_blocks=True)
    raise ValueError(name)
