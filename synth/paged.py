"""A packed synthetic case moved into a paged K/V/position pool (data layout
only).  Physical pages are assigned in a seeded random order, and spare
pages hold random bits, so a kernel that reads the wrong page reads garbage.

Pool rows: layer l, physical page p, slot t, KV head g sits at
  l*layer_stride + p*page_stride + t*token_stride + g*head_stride
with token-major pages ([page][slot][head]) or head-major pages
([page][head][slot]).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .cases import SEED_BASE, Case


@dataclass
class PagedPool:
    page_size: int
    num_pages: int
    max_pages: int
    page_stride: int
    token_stride: int
    head_stride: int
    layer_stride: int
    table: torch.Tensor          # int32 [S, max_pages] (device)
    k: torch.Tensor              # int16 [rows, d]
    v: torch.Tensor | None       # int16 [rows, d]
    pos: torch.Tensor            # int32 [rows]

    def strides(self):
        return (self.page_stride, self.token_stride, self.head_stride, self.layer_stride)

    def unit_rows(self, s: int, l: int, g: int, n: int) -> np.ndarray:
        """Pool rows of tokens 0..n-1 of unit (s, l, g) (vectorised)."""
        i = np.arange(n, dtype=np.int64)
        tab = self.table[s].cpu().numpy().astype(np.int64)
        page = tab[i // self.page_size]
        return (l * self.layer_stride + g * self.head_stride + page * self.page_stride
                + (i % self.page_size) * self.token_stride)


def empty_pool(S, L, Hkv, d, page_size, pages_needed, head_major=False, spare=3, seed=0,
               device="cpu", with_values=True, max_pages=None) -> PagedPool:
    """A pool of sum(pages_needed) + spare pages filled with random bits and
    a random page table (sequence s owns pages_needed[s] distinct pages)."""
    num_pages = int(sum(pages_needed)) + spare
    max_pages = max(1, max(pages_needed) if max_pages is None else max_pages)
    g = np.random.default_rng([SEED_BASE, 77, seed])
    perm = g.permutation(num_pages)
    table = np.zeros((S, max_pages), dtype=np.int32)
    o = 0
    for s in range(S):
        table[s, :pages_needed[s]] = perm[o:o + pages_needed[s]]
        table[s, pages_needed[s]:] = perm[-1] if spare else 0   # entries past the end: unused
        o += pages_needed[s]
    P = page_size
    page_rows = P * Hkv
    rows = L * num_pages * page_rows
    gen = torch.Generator(device=device)
    gen.manual_seed(int(g.integers(1 << 62)))
    k = torch.randint(-32768, 32767, (rows, d), dtype=torch.int16, device=device, generator=gen)
    v = torch.randint(-32768, 32767, (rows, d), dtype=torch.int16, device=device,
                      generator=gen) if with_values else None
    pos = torch.randint(-(1 << 30), 1 << 30, (rows,), dtype=torch.int32, device=device,
                        generator=gen)
    tok, head = (1, P) if head_major else (Hkv, 1)
    return PagedPool(P, num_pages, max_pages, page_rows, tok, head, num_pages * page_rows,
                     torch.as_tensor(table, device=device), k, v, pos)


def paged_from_case(case: Case, page_size: int, head_major=False, spare=3, seed=0) -> PagedPool:
    """The case's keys, values and positions scattered into a fresh pool."""
    S, L, H = case.num_seqs, case.shape.num_layers, case.shape.num_kv_heads
    P = page_size
    need = [(case.seq_len(s) + P - 1) // P for s in range(S)]
    pool = empty_pool(S, L, H, case.shape.head_dim, P, need, head_major, spare, seed,
                      case.k.device, case.v is not None)
    for s in range(S):
        n = case.seq_len(s)
        if n == 0:
            continue
        for l in range(L):
            for g in range(H):
                start, _ = case.unit_rows(s, l, g)
                dst = torch.as_tensor(pool.unit_rows(s, l, g, n), device=case.k.device)
                pool.k[dst] = case.k[start:start + n]
                if case.v is not None:
                    pool.v[dst] = case.v[start:start + n]
                pool.pos[dst] = case.k_pos[start:start + n]
    return pool
