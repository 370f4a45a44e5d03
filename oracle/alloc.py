"""Reference KV-pool allocators (oracle; test infrastructure only).

COLD pool — "Paged KV cache" page, sections "How it works" and "Code": a pool
of fixed-size blocks with a LIFO free stack and per-block reference counts;
one block table and length per sequence; ``append`` reserves a slot for one
more token (a new block when the previous one is full, copy-on-write when the
partially filled last block is shared); ``fork`` shares every block without
copying; ``release`` drops every reference.  The page fixes the block size at
16; here it is a parameter P (the GraniKV paper uses P = 1 for its COLD pool,
its Section 3.3, and sweeps P in {1, 4, 16}, its Appendix B.6).

HOT pool — GraniKV paper, Section 3.2: a contiguous allocator over a region
reserved up front.  Each prefix gets one contiguous range of Lp token slots;
the caller keeps its base index.  A slab whose reference count drops to zero
becomes evictable; eviction (least recently released first) returns
[base, base + Lp) to a free list and merges it with neighbouring free ranges.
A prefix either occupies its whole range or is absent.  Admission that finds
no room is reported to the caller, who then stores the prefix in the COLD pool
(paper, Appendix B.10).

Readings where the pages are silent (each also listed in the design notes):
  * Free stack order: a new pool pops pages 0, 1, 2, ... (the page's
    constructor pushes n-1 ... 0).  A caller-given ``free_order`` is the pop
    order instead (used for shuffled slots).
  * ``release`` retires the sequence id; later operations on it are a state
    error (so a double release is detected).
  * Failed allocations leave every piece of state unchanged (the page's
    ``alloc`` fails before any mutation; copy-on-write allocates before it
    decrements).
  * HOT placement is first-fit by ascending base.  When nothing fits, the pool
    first checks whether evicting every unreferenced slab would make room; if
    not it fails without evicting.  Otherwise it evicts unreferenced slabs one
    at a time, least recently released first, retrying first-fit after each.
  * ``fork`` of a sequence in the COLD pool does not touch HOT refcounts; the
    caller increments the slab of the request's group itself.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple


class PoolError(Exception):
    """Base class; ``code`` mirrors the status codes of the C interface."""
    code = -1


class InvalidArgument(PoolError):
    code = -1


class OutOfMemory(PoolError):
    code = -2


class StateError(PoolError):
    code = -3


@dataclass
class Seq:
    table: List[int] = field(default_factory=list)
    length: int = 0
    live: bool = True


class ColdPool:
    """Block pool with refcounts, copy-on-write and slot mapping."""

    def __init__(self, num_pages: int, page_size: int, free_order: Optional[List[int]] = None):
        if num_pages < 0 or page_size < 1:
            raise InvalidArgument("bad pool shape")
        self.page_size = int(page_size)
        self.num_pages = int(num_pages)
        self.ref = [0] * self.num_pages
        if free_order is None:
            pops = list(range(self.num_pages))
        else:
            pops = [int(x) for x in free_order]
            if sorted(pops) != list(range(self.num_pages)):
                raise InvalidArgument("free_order must be a permutation of the pages")
        # Stored bottom -> top; the top (end of the list) is popped first.
        self.free: List[int] = list(reversed(pops))
        self.seqs: Dict[int, Seq] = {}
        self.next_id = 0

    # -- page ownership ----------------------------------------------------
    def _take_page(self) -> int:
        """Hand out the page on top of the free stack, owned once."""
        page = self.free.pop()
        self.ref[page] = 1
        return page

    def _drop_page(self, page: int) -> None:
        """One owner fewer; a page nobody owns goes back on the free stack."""
        if self.ref[page] <= 0:
            raise StateError(f"decref of free page {page}")
        self.ref[page] -= 1
        if self.ref[page] == 0:
            self.free.append(page)

    def num_free(self) -> int:
        return len(self.free)

    def _seq(self, sid: int) -> Seq:
        s = self.seqs.get(sid)
        if s is None or not s.live:
            raise StateError(f"unknown or released sequence {sid}")
        return s

    # -- sequence operations --------------------------------------------
    def seq_new(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = Seq()
        return sid

    def append(self, sid: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Slot of the sequence's next token; returns (slot, copy-on-write pair or None).

        The token at position ``length`` lives in page ``length // P`` of the
        sequence, row ``length % P``.  The sequence must hold that page alone
        before the token is written: a page it does not have yet, or one that
        a fork still shares, is replaced by a page from the free stack (the
        shared page keeps its other owners and the caller copies its rows).
        """
        s = self._seq(sid)
        P = self.page_size
        page_index, row = divmod(s.length, P)
        starts_page = page_index == len(s.table)
        shared = not starts_page and self.ref[s.table[page_index]] > 1
        cow = None
        if starts_page or shared:
            if not self.free:
                raise OutOfMemory("COLD pool exhausted" + (" (copy-on-write)" if shared else ""))
            page = self._take_page()
            if shared:
                old = s.table[page_index]
                s.table[page_index] = page
                self._drop_page(old)
                cow = (old, page)
            else:
                s.table.append(page)
        s.length += 1
        return s.table[page_index] * P + row, cow

    def append_batch(self, seqs: List[int]):
        """Single appends in array order; stops at the first failure.

        Returns (slots, cow_pairs, n_done, error-or-None)."""
        slots, cows = [], []
        for i, sid in enumerate(seqs):
            try:
                slot, cow = self.append(int(sid))
            except PoolError as e:
                return slots, cows, i, e
            slots.append(slot)
            if cow is not None:
                cows.append(cow)
        return slots, cows, len(seqs), None

    def fork(self, sid: int) -> int:
        """A new sequence with the same history: every page gains an owner."""
        s = self._seq(sid)
        nid = self.seq_new()
        self.seqs[nid] = Seq(list(s.table), s.length)
        for page in s.table:
            self.ref[page] += 1
        return nid

    def release(self, sid: int) -> None:
        """The sequence gives up every page it owns (in table order) and its id."""
        s = self._seq(sid)
        for page in s.table:
            self._drop_page(page)
        s.table, s.length, s.live = [], 0, False

    # -- views -------------------------------------------------------------
    def block_table(self, sid: int) -> List[int]:
        return list(self._seq(sid).table)

    def length(self, sid: int) -> int:
        return self._seq(sid).length

    def state(self):
        """Everything that must match bit for bit between implementations."""
        live = {sid: (tuple(s.table), s.length) for sid, s in sorted(self.seqs.items()) if s.live}
        return {"ref": list(self.ref), "free": list(self.free), "seqs": live, "next_id": self.next_id}


@dataclass
class Slab:
    length: int
    ref: int
    lru: int = -1      # tick stamped when ref dropped to 0; -1 while referenced


class HotPool:
    """Contiguous first-fit slab allocator with LRU eviction of unreferenced slabs."""

    def __init__(self, capacity: int):
        if capacity < 0:
            raise InvalidArgument("negative capacity")
        self.capacity = int(capacity)
        self.free: List[Tuple[int, int]] = [(0, self.capacity)] if capacity > 0 else []
        self.slabs: Dict[int, Slab] = {}
        self.tick = 0

    def _insert_free(self, base: int, length: int, free=None) -> List[Tuple[int, int]]:
        """Return the free list with [base, base+length) added and neighbours merged."""
        ranges = sorted((self.free if free is None else free) + [(base, length)])
        merged: List[Tuple[int, int]] = []
        for b, n in ranges:
            if merged and merged[-1][0] + merged[-1][1] == b:
                merged[-1] = (merged[-1][0], merged[-1][1] + n)
            else:
                merged.append((b, n))
        return merged

    def _first_fit(self, lp: int) -> Optional[int]:
        for i, (b, n) in enumerate(self.free):
            if n >= lp:
                if n == lp:
                    del self.free[i]
                else:
                    self.free[i] = (b + lp, n - lp)
                return b
        return None

    def _evict(self, base: int) -> None:
        s = self.slabs.pop(base)
        self.free = self._insert_free(base, s.length)

    def _lru_order(self) -> List[int]:
        cands = [(s.lru, base) for base, s in self.slabs.items() if s.ref == 0]
        return [base for _, base in sorted(cands)]

    def alloc(self, lp: int) -> int:
        if lp <= 0:
            raise InvalidArgument("prefix length must be positive")
        order = self._lru_order()
        # Would evicting everything evictable make room?  If not, fail unchanged.
        free = list(self.free)
        for base in order:
            free = self._insert_free(base, self.slabs[base].length, free)
        if not any(n >= lp for _, n in free):
            raise OutOfMemory("HOT pool has no contiguous range of that length")
        while True:
            b = self._first_fit(lp)
            if b is not None:
                self.slabs[b] = Slab(lp, 1)
                return b
            self._evict(order.pop(0))

    def _slab(self, base: int) -> Slab:
        s = self.slabs.get(base)
        if s is None:
            raise StateError(f"no slab at base {base}")
        return s

    def incref(self, base: int) -> None:
        s = self._slab(base)
        s.ref += 1
        s.lru = -1

    def decref(self, base: int) -> None:
        s = self._slab(base)
        if s.ref <= 0:
            raise StateError(f"decref of unreferenced slab {base}")
        s.ref -= 1
        if s.ref == 0:
            s.lru = self.tick
            self.tick += 1

    def evict_unreferenced(self) -> int:
        order = self._lru_order()
        for base in order:
            self._evict(base)
        return len(order)

    def free_tokens(self) -> int:
        return sum(n for _, n in self.free)

    def state(self):
        slabs = [(b, s.length, s.ref, s.lru) for b, s in sorted(self.slabs.items())]
        return {"free": list(self.free), "slabs": slabs, "tick": self.tick}
