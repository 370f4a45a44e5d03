"""numpy mirror of the device KV pools (oracle; test infrastructure only).

Layouts (design readings of the pages, also listed in the design notes):
  * HOT (GraniKV paper, Section 3.2): a prefix admitted at token slot ``base``
    with length Lp stores layer l's head h at the stride the paper gives,
    base + l * Lp * Hkv + h * Lp in rows, with the slab of all L layers
    starting at row base * Hkv * L: element (l, t, h, c) lives at
    ((base * Hkv * L + l * Lp * Hkv + h * Lp) + t) * d + c.  Each head's
    prefix in each layer is one dense [Lp, d] matrix.
  * COLD ("Paged KV cache" page, "How it works"): the slot of token t of a
    sequence is table[t // P] * P + t % P; a slot's row holds all KV heads,
    and the pool is layer-major with the same slots in every layer: element
    (l, slot, h, c) at ((l * num_slots + slot) * Hkv + h) * d + c.  A
    copy-on-write copy applies to the page in every layer.

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


def hot_offset(base: int, lp: int, hkv: int, d: int, t: int, h: int, layer: int = 0, num_layers: int = 1) -> int:
    """Element offset of (layer, token t, head h, column 0) of a HOT slab."""
    return ((base * hkv * num_layers + layer * lp * hkv + h * lp) + t) * d


def cold_slot(table: Sequence[int], t: int, page_size: int) -> int:
    """Physical slot of logical token t of a sequence."""
    return int(table[t // page_size]) * page_size + t % page_size


class PoolMirror:
    def __init__(self, hot_capacity: int, cold_slots: int, hkv: int, d: int, np_dtype, num_layers: int = 1):
        self.hkv, self.d, self.num_layers = hkv, d, num_layers
        self.hot_capacity, self.cold_slots = hot_capacity, cold_slots
        self.k_hot = np.zeros(hot_capacity * hkv * d * num_layers, dtype=np_dtype)
        self.v_hot = np.zeros(hot_capacity * hkv * d * num_layers, dtype=np_dtype)
        self.k_cold = np.zeros(num_layers * cold_slots * hkv * d, dtype=np_dtype)
        self.v_cold = np.zeros(num_layers * cold_slots * hkv * d, dtype=np_dtype)

    def _cold(self, layer: int):
        n = self.cold_slots * self.hkv * self.d
        return self.k_cold[layer * n:(layer + 1) * n], self.v_cold[layer * n:(layer + 1) * n]

    def hot_write(self, k_src: np.ndarray, v_src: np.ndarray, base: int, layer: int = 0) -> None:
        """Store one layer of a prefix's [Lp, Hkv, d] K/V into its slab."""
        lp = k_src.shape[0]
        hkv, d = self.hkv, self.d
        for h in range(hkv):
            for t in range(lp):
                o = hot_offset(base, lp, hkv, d, t, h, layer, self.num_layers)
                self.k_hot[o:o + d] = k_src[t, h]
                self.v_hot[o:o + d] = v_src[t, h]

    def reshape_and_cache(self, k_new: np.ndarray, v_new: np.ndarray, slots: Sequence[int], layer: int = 0) -> None:
        """Write token i's [Hkv, d] K/V row at slots[i] of one layer; slots outside the pool are skipped."""
        row = self.hkv * self.d
        kc, vc = self._cold(layer)
        for i, s in enumerate(slots):
            s = int(s)
            if 0 <= s < self.cold_slots:
                kc[s * row:(s + 1) * row] = k_new[i].reshape(-1)
                vc[s * row:(s + 1) * row] = v_new[i].reshape(-1)

    def copy_blocks(self, pairs: Sequence[Sequence[int]], page_size: int) -> None:
        """Copy whole pages src -> dst (K and V) in every layer, in pair order."""
        span = page_size * self.hkv * self.d
        for layer in range(self.num_layers):
            kc, vc = self._cold(layer)
            for src, dst in pairs:
                src, dst = int(src), int(dst)
                kc[dst * span:(dst + 1) * span] = kc[src * span:(src + 1) * span]
                vc[dst * span:(dst + 1) * span] = vc[src * span:(src + 1) * span]

    def gather_prefix(self, base: int, lp: int, layer: int = 0):
        hkv, d = self.hkv, self.d
        k = np.empty((lp, hkv, d), dtype=self.k_hot.dtype)
        v = np.empty_like(k)
        for h in range(hkv):
            o = hot_offset(base, lp, hkv, d, 0, h, layer, self.num_layers)
            k[:, h] = self.k_hot[o:o + lp * d].reshape(lp, d)
            v[:, h] = self.v_hot[o:o + lp * d].reshape(lp, d)
        return k, v

    def gather_suffix(self, table: Sequence[int], length: int, page_size: int, layer: int = 0):
        hkv, d = self.hkv, self.d
        row = hkv * d
        kc, vc = self._cold(layer)
        k = np.empty((length, hkv, d), dtype=self.k_cold.dtype)
        v = np.empty_like(k)
        for t in range(length):
            s = cold_slot(table, t, page_size)
            k[t] = kc[s * row:(s + 1) * row].reshape(hkv, d)
            v[t] = vc[s * row:(s + 1) * row].reshape(hkv, d)
        return k, v
