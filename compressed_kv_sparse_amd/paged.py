"""Paged compressed caches ("vLLM DeepSeek V4 サポート", KV cache memory
management): one logical block covers 256 token positions on every compressed
layer, so a block holds 64 compressed rows of a c4a layer (and the 64 indexer
rows of the same positions) or 2 rows of a c128a layer.  The library reads
and writes those rows through a per-layer block table (ckv_layer_cache
.block_table); this module owns the pages.

Pages of equal size share one pool across layers, which gives three page
sizes for a stack of c4a and c128a layers: c4a K=V pages (64 rows), c4a
indexer pages (64 indexer rows) and c128a K=V pages (2 rows).  A c4a layer's
K=V and indexer rows of one block sit at the same page index of their two
pools, so the two c4a pools share one free list; c128a pages have their own.
The raw window and the compressor state are not paged: the library keeps them
as per-sequence rings keyed by position, the sliding-window form the page
describes for the compressor state.

Host logic only (free lists and tables); device memory comes from torch.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

BLOCK_TOKENS = 256


def rows_per_block(ratio: int) -> int:
    """Compressed rows of one 256-position block (64 for c4a, 2 for c128a)."""
    if ratio not in (4, 128):
        raise ValueError("only compressed layers (ratio 4 or 128) are paged")
    return BLOCK_TOKENS // ratio


class FreeList:
    """Page indices [0, n) handed out lowest first (after a release, the
    released pages come back first)."""

    def __init__(self, n: int):
        if n < 1:
            raise ValueError("a pool needs at least one page")
        self.n = n
        self._free: List[int] = list(range(n - 1, -1, -1))

    def alloc(self) -> int:
        if not self._free:
            raise MemoryError("page pool exhausted")
        return self._free.pop()

    def release(self, pages) -> None:
        for p in sorted((int(x) for x in pages), reverse=True):
            if not 0 <= p < self.n:
                raise ValueError(f"page {p} is not in the pool")
            self._free.append(p)

    @property
    def n_free(self) -> int:
        return len(self._free)


class PagePools:
    """The page pools of one GPU, by page size.

    kv_row_bytes is the stored K=V row (ckv_row_bytes), idx_row_bytes the
    stored indexer row (ckv_idx_row_bytes); pages_c4a / pages_c128a the pages
    of each id space (0: none).  Layers made with ``pages=`` this object take
    their pools from here."""

    def __init__(self, *, kv_row_bytes: int, idx_row_bytes: int = 0, pages_c4a: int = 0, pages_c128a: int = 0,
                 device="cuda"):
        dev = torch.device(device)
        self.kv_row_bytes, self.idx_row_bytes = kv_row_bytes, idx_row_bytes
        self.pools: Dict[str, torch.Tensor] = {}
        self.free: Dict[int, FreeList] = {}
        if pages_c4a:
            self.pools["c4a_kv"] = torch.zeros((pages_c4a, 64, kv_row_bytes), dtype=torch.uint8, device=dev)
            if idx_row_bytes:
                self.pools["c4a_idx"] = torch.zeros((pages_c4a, 64, idx_row_bytes), dtype=torch.uint8, device=dev)
            self.free[4] = FreeList(pages_c4a)
        if pages_c128a:
            self.pools["c128a_kv"] = torch.zeros((pages_c128a, 2, kv_row_bytes), dtype=torch.uint8, device=dev)
            self.free[128] = FreeList(pages_c128a)

    def page_sizes(self) -> Dict[str, int]:
        """Bytes of one page of each pool."""
        return {k: int(v.shape[1] * v.shape[2]) for k, v in self.pools.items()}

    def kv_pool(self, ratio: int) -> torch.Tensor:
        return self.pools["c4a_kv" if ratio == 4 else "c128a_kv"]

    def idx_pool(self) -> Optional[torch.Tensor]:
        return self.pools.get("c4a_idx")

    def n_pages(self, ratio: int) -> int:
        return self.free[ratio].n


class BlockTable:
    """One layer's block table: table[b, j] = the page of block j of sequence
    b (positions 256 j .. 256 j + 255), or -1.  The device copy is what the
    library reads; map / release update both."""

    def __init__(self, free: FreeList, batch: int, max_blocks: int, device="cuda"):
        self.free = free
        self.host = np.full((batch, max_blocks), -1, dtype=np.int32)
        self.dev = torch.full((batch, max_blocks), -1, dtype=torch.int32, device=torch.device(device))

    def map_blocks(self, b: int, n_blocks: int, order=None) -> None:
        """Give blocks 0 .. n_blocks - 1 of sequence b a page each (those that
        have none).  ``order``: optional pages to take instead of the free
        list's (they must be free; tests use it to scatter the pages)."""
        row = self.host[b]
        if n_blocks > row.shape[0]:
            raise ValueError("blocks beyond the table (comp_cap)")
        todo = [j for j in range(n_blocks) if row[j] < 0]
        if order is not None:
            order = [int(p) for p in order][:len(todo)]
            if len(order) < len(todo):
                raise ValueError("not enough pages given")
            taken = set(order)
            if len(taken) != len(order):
                raise ValueError("a page given twice")
            free = self.free._free
            missing = taken - set(free)
            if missing:
                raise ValueError(f"pages not free: {sorted(missing)[:4]}")
            self.free._free = [p for p in free if p not in taken]
            for j, p in zip(todo, order):
                row[j] = p
        else:
            for j in todo:
                row[j] = self.free.alloc()
        if todo:
            self.dev[b].copy_(torch.from_numpy(row.copy()))

    def release(self, b: int) -> None:
        row = self.host[b]
        used = row[row >= 0]
        self.free.release(used)
        row[:] = -1
        self.dev[b].fill_(-1)
