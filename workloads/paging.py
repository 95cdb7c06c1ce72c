"""Seeded paged layouts of a packed K/V cache (storage only: no part of the method
is computed here).

A paged cache keeps every sequence's tokens in fixed-size pages of a shared pool;
a block table row per sequence lists its pages in token order.  ``page_layout``
draws which pool page holds which (sequence, page) from a seeded permutation, so
consecutive pages of a sequence are scattered over the pool.  The pool has two
spare pages; the first is the padding entry of every block-table row past a
sequence's last page.  ``to_pages`` copies packed rows into such a pool and fills
every slot that holds no token with NaN, so a read of a wrong row shows up in
the results instead of passing unnoticed (and every block-table entry is a valid
page, so even such a read stays inside the pool).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import torch

from .gen import _perm


@dataclass
class PageLayout:
    page_size: int
    n_pages: int                  # pool pages, spares included
    block_table: torch.Tensor     # int32 [batch, max_pages] (CPU)
    seqlens_k: List[int]

    @property
    def pool_rows(self) -> int:
        return self.n_pages * self.page_size


def page_layout(seqlens_k, page_size: int, seed: int, max_pages: int = 0) -> PageLayout:
    need = [-(-int(n) // page_size) for n in seqlens_k]
    max_pages = max(max_pages, max(need), 1)
    n_used = sum(need)
    n_pages = n_used + 2
    perm = _perm(n_pages, seed, f"pages:{page_size}").to(torch.int32)
    pad = perm[n_used].item()                     # the first spare page
    bt = torch.full((len(seqlens_k), max_pages), pad, dtype=torch.int32)
    o = 0
    for b, m in enumerate(need):
        bt[b, :m] = perm[o:o + m]
        o += m
    return PageLayout(page_size, n_pages, bt, [int(n) for n in seqlens_k])


def token_rows(layout: PageLayout) -> torch.Tensor:
    """Pool row of every packed token (int64 [sum N_b])."""
    rows = []
    ps = layout.page_size
    for b, n in enumerate(layout.seqlens_k):
        t = torch.arange(n)
        rows.append(layout.block_table[b, t // ps].long() * ps + t % ps)
    return torch.cat(rows) if rows else torch.zeros(0, dtype=torch.long)


def to_pages(x: torch.Tensor, layout: PageLayout) -> torch.Tensor:
    """Packed [sum N_b, h, d] -> pool [n_pages * page_size, h, d] (same device and dtype)."""
    pool = torch.full((layout.pool_rows,) + tuple(x.shape[1:]), float("nan"), dtype=x.dtype, device=x.device)
    pool[token_rows(layout).to(x.device)] = x
    return pool


def from_pages(pool: torch.Tensor, layout: PageLayout) -> torch.Tensor:
    """Pool -> packed [sum N_b, h, d]."""
    return pool[token_rows(layout).to(pool.device)]
