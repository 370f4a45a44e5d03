"""numpy mirror of the device KV pools (oracle; test infrastructure only).

Layouts (design readings of the pages, also listed in the design notes):
  * HOT (GraniKV paper, Section 3.2): a prefix admitted at token slot ``base``
    with length Lp stores head h's rows at the stride the paper gives,
    base + h * Lp (in token slots, one layer, times Hkv for the slab start):
    element (t, h, c) lives at ((base * Hkv + h * Lp) + t) * d + c.  Each
    head's prefix is one dense [Lp, d] matrix.
  * COLD ("Paged KV cache" page, "How it works"): the slot of token t of a
    sequence is table[t // P] * P + t % P; a slot's row holds all KV heads,
    element (slot, h, c) at (slot * Hkv + h) * d + c.

Storage keeps the input representation (bf16 bit patterns as uint16, or
float32) so device pools can be compared byte for byte.

Pinned by ``tests/test_oracle_pools.py``: the "Paged KV cache" page's
block-table picture written and read back through the mirror (tokens 0-15 in
block 3, 16-31 in block 0, 32-40 in block 4), a hand-computed HOT offset and
slab placement, a hand-worked two-page ``copy_blocks`` (pair order, all heads),
slots outside the pool skipped, and the copy-on-write invariant: after fork +
append at page size 16 the pre-fork rows and the HOT slab are byte-identical.
``tests/test_oracle_attention.py`` also checks that attention read back
through the mirror equals attention over the drawn tokens.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def hot_offset(base: int, lp: int, hkv: int, d: int, t: int, h: int) -> int:
    """Element offset of (token t, head h, column 0) of a HOT slab."""
    return ((base * hkv + h * lp) + t) * d


def cold_slot(table: Sequence[int], t: int, page_size: int) -> int:
    """Physical slot of logical token t of a sequence."""
    return int(table[t // page_size]) * page_size + t % page_size


class PoolMirror:
    def __init__(self, hot_capacity: int, cold_slots: int, hkv: int, d: int, np_dtype):
        self.hkv, self.d = hkv, d
        self.hot_capacity, self.cold_slots = hot_capacity, cold_slots
        self.k_hot = np.zeros(hot_capacity * hkv * d, dtype=np_dtype)
        self.v_hot = np.zeros(hot_capacity * hkv * d, dtype=np_dtype)
        self.k_cold = np.zeros(cold_slots * hkv * d, dtype=np_dtype)
        self.v_cold = np.zeros(cold_slots * hkv * d, dtype=np_dtype)

    def hot_write(self, k_src: np.ndarray, v_src: np.ndarray, base: int) -> None:
        """Store a prefix's [Lp, Hkv, d] K/V into its slab."""
        lp = k_src.shape[0]
        hkv, d = self.hkv, self.d
        for h in range(hkv):
            for t in range(lp):
                o = hot_offset(base, lp, hkv, d, t, h)
                self.k_hot[o:o + d] = k_src[t, h]
                self.v_hot[o:o + d] = v_src[t, h]

    def reshape_and_cache(self, k_new: np.ndarray, v_new: np.ndarray, slots: Sequence[int]) -> None:
        """Write token i's [Hkv, d] K/V row at slots[i]; slots outside the pool are skipped."""
        row = self.hkv * self.d
        for i, s in enumerate(slots):
            s = int(s)
            if 0 <= s < self.cold_slots:
                self.k_cold[s * row:(s + 1) * row] = k_new[i].reshape(-1)
                self.v_cold[s * row:(s + 1) * row] = v_new[i].reshape(-1)

    def copy_blocks(self, pairs: Sequence[Sequence[int]], page_size: int) -> None:
        """Copy whole pages src -> dst (K and V), in pair order."""
        span = page_size * self.hkv * self.d
        for src, dst in pairs:
            src, dst = int(src), int(dst)
            self.k_cold[dst * span:(dst + 1) * span] = self.k_cold[src * span:(src + 1) * span]
            self.v_cold[dst * span:(dst + 1) * span] = self.v_cold[src * span:(src + 1) * span]

    def gather_prefix(self, base: int, lp: int):
        hkv, d = self.hkv, self.d
        k = np.empty((lp, hkv, d), dtype=self.k_hot.dtype)
        v = np.empty_like(k)
        for h in range(hkv):
            o = hot_offset(base, lp, hkv, d, 0, h)
            k[:, h] = self.k_hot[o:o + lp * d].reshape(lp, d)
            v[:, h] = self.v_hot[o:o + lp * d].reshape(lp, d)
        return k, v

    def gather_suffix(self, table: Sequence[int], length: int, page_size: int):
        hkv, d = self.hkv, self.d
        row = hkv * d
        k = np.empty((length, hkv, d), dtype=self.k_cold.dtype)
        v = np.empty_like(k)
        for t in range(length):
            s = cold_slot(table, t, page_size)
            k[t] = self.k_cold[s * row:(s + 1) * row].reshape(hkv, d)
            v[t] = self.v_cold[s * row:(s + 1) * row].reshape(hkv, d)
        return k, v
