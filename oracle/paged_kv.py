"""Paged KV cache: the oracle's view of a cache kept in fixed-size pages.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never calls it.

"Baseten optimizes Qwen3-ASR 1.7B", section "Our optimized Qwen3-ASR stack":
the serving stack starts from vLLM's transcription endpoint and batches 30 s
windows through the model.  vLLM's engine keeps every sequence's K/V in
fixed-size pages of one shared pool, addressed through a per-sequence page
table, so that sequences of very different lengths share HBM without each
reserving its maximum length.  The page names the engine, not a layout; the
readings taken here:

* The pool holds num_pages pages; page p, kv head g, row r of K is
  k[p][g][r][0 .. d) (head-major inside a page, like the contiguous cache
  inside a slot).  V has the same layout.
* Slot s owns the table row table[s][0 .. pages_per_seq): its position t lives
  in page table[s][t // P], row t % P (P = page_size).  The largest length of a
  slot is pages_per_seq * P.
* Page ids are the caller's: several slots may name the same page (a shared
  prompt prefix), as long as no call appends into a page another live slot
  reads.  A call that needs a position whose page id is outside
  [0, num_pages) sets STATUS_BAD_PAGE: that sequence's output rows, length and
  appended rows are unspecified (nothing outside the pool is read or
  written); its other sequences are unaffected.

Every operation on a paged cache is the same operation on the contiguous
cache the table describes (gather), with the rows the operation appended
written back to their pages (scatter).  That is the whole definition: the
arithmetic is the contiguous oracle's.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .attn_block import E4M3, KVCache

STATUS_BAD_PAGE = 16   # a needed position's page id lies outside the pool: that sequence skipped


@dataclass
class PagedKV:
    """One layer's paged cache: K and V pools [num_pages][nkv][P][d] of codes, the page table
    [batch_cap][pages_per_seq] and the committed lengths [batch_cap]."""
    k: np.ndarray
    v: np.ndarray
    table: np.ndarray
    lens: np.ndarray
    dtype: str
    status: int = 0

    @classmethod
    def empty(cls, num_pages, n_kv_heads, page_size, head_dim, table, dtype):
        shape = (num_pages, n_kv_heads, page_size, head_dim)
        ct = np.uint8 if dtype == E4M3 else np.uint16
        table = np.asarray(table, np.int64)
        return cls(np.zeros(shape, ct), np.zeros(shape, ct), table, np.zeros(table.shape[0], np.int64), dtype)

    @property
    def page_size(self) -> int:
        return self.k.shape[2]

    @property
    def pages_per_seq(self) -> int:
        return self.table.shape[1]

    @property
    def capacity(self) -> int:
        return self.page_size * self.pages_per_seq

    def copy(self) -> "PagedKV":
        return PagedKV(self.k.copy(), self.v.copy(), self.table.copy(), self.lens.copy(), self.dtype, self.status)

    def locate(self, s: int, t: int):
        """(page, row) of position t of slot s; page None when the table entry is outside the pool."""
        p = int(self.table[s, t // self.page_size])
        if not 0 <= p < self.k.shape[0]:
            return None, t % self.page_size
        return p, t % self.page_size

    def pages_ok(self, s: int, upto: int) -> bool:
        """Whether every position < upto of slot s has a page in the pool."""
        return all(self.locate(s, t)[0] is not None for t in range(0, upto, self.page_size))

    def gather(self) -> KVCache:
        """The contiguous cache [batch_cap][nkv][capacity][d] the table describes (positions whose
        page id lies outside the pool read as zero codes)."""
        B = self.table.shape[0]
        nkv, d, P = self.k.shape[1], self.k.shape[3], self.page_size
        c = KVCache.empty(B, nkv, self.capacity, d, self.dtype)
        for s in range(B):
            for j in range(self.pages_per_seq):
                p = int(self.table[s, j])
                if 0 <= p < self.k.shape[0]:
                    c.k[s, :, j * P:(j + 1) * P] = self.k[p]
                    c.v[s, :, j * P:(j + 1) * P] = self.v[p]
        c.lens[:] = self.lens
        return c

    def scatter_rows(self, c: KVCache, s: int, t0: int, t1: int) -> None:
        """Write positions t0 .. t1 - 1 of slot s of the contiguous cache c back to their pages."""
        for t in range(t0, t1):
            p, r = self.locate(s, t)
            self.k[p, :, r] = c.k[s, :, t]
            self.v[p, :, r] = c.v[s, :, t]


def on_pages(pkv: PagedKV, slots, rows, op):
    """Run op(contiguous cache) -> output on the cache the table describes, then store the rows
    it appended into their pages.  slots: the slot of each sequence of the call; rows: the rows
    each appends.  A sequence that needs a page outside the pool makes the call set
    STATUS_BAD_PAGE; its outputs, length and appended rows are unspecified (here: NaN
    outputs, pages and length left as they were)."""
    slots = [int(s) for s in slots]
    rows = [int(n) for n in rows]
    bad = [not pkv.pages_ok(s, min(int(pkv.lens[s]) + n, pkv.capacity)) for s, n in zip(slots, rows)]
    c = pkv.gather()
    before = c.lens.copy()
    out = op(c)
    for b, s in enumerate(slots):
        if bad[b]:
            pkv.status |= STATUS_BAD_PAGE
            continue
        pkv.scatter_rows(c, s, int(before[s]), int(c.lens[s]))
        pkv.lens[s] = c.lens[s]
    pkv.status |= c.status
    if out is not None:
        out = np.array(out, np.float64, copy=True)
        r = 0
        for b, n in enumerate(rows):
            if bad[b]:
                out.reshape(-1, out.shape[-1])[r:r + n] = np.nan
            r += n
    return out
