"""Runs drawn workloads through the oracle allocators and pool mirror.

Test infrastructure only.  It fixes the order of allocator operations that
both implementations follow, so slots, block tables, copy-on-write pairs and
allocator state can be compared bit for bit:

Single decode step (one step of the "Paged KV cache" page's "How it works"
list, with the GraniKV paper's HOT prefix):
  1. Each prefix group's slab is allocated first-fit in group order; the slab
     holds one reference per member request (alloc, then one incref per
     additional member).
  2. Every request gets a new COLD sequence (ids 0..B-1).
  3. Setup: the first Ls_b - 1 suffix tokens are appended request-major
     (all of request 0's, then request 1's, ...), and written with
     reshape_and_cache.
  4. The step: one append per request in ascending id (the token being
     decoded), then copy-on-write copies, then reshape_and_cache of the new
     token, then attention over Lp_b + Ls_b tokens.

Multi-step run over a multi-prefix workload (groups of requests, each group
with its own prefix; the paper's heterogeneous multi-agent setting, Section
4.5 Table 4 and Appendix B.8b): after the setup, for each step s:
  * at ``fork_step``, before the appends, the first request of every group
    forks (COLD fork, plus one HOT reference); children get the next ids and
    share the parent's logical history;
  * at ``release_step``, before the appends, those fork parents are released
    (COLD release, minus one HOT reference);
  * every live request appends one token (ascending id); copy-on-write pairs
    are copied, then the new tokens are written;
  * attention covers every live request.
At the end every live request is released and unreferenced slabs evicted.

Pinned by ``tests/test_oracle_driver.py`` (refcounts against live tables, HOT
refcounts against live members, histories built from the draws, the fork and
release schedule, teardown, and both reference forms against the flat oracle)
and, for the single step, by the page-size and slot-order invariance and the
pool-mirror pins.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from .alloc import ColdPool, HotPool
from .attention import attend, attend_shared_prefix, widen, NEG_INF
from .pools import PoolMirror


def admit_prefixes(hot: HotPool, wl) -> List[int]:
    members = np.bincount(wl.group_of[wl.group_of >= 0], minlength=len(wl.group_prefix_len))
    bases = []
    for g, lp in enumerate(wl.group_prefix_len):
        base = hot.alloc(int(lp))
        for _ in range(int(members[g]) - 1):
            hot.incref(base)
        bases.append(base)
    return bases


def _np_dtype(wl):
    return np.uint16 if wl.cfg.dtype == "bf16" else np.float32


@dataclass
class SingleStep:
    hot: HotPool
    cold: ColdPool
    bases: List[int]
    seqs: List[int]
    setup_slots: List[int]
    step_slots: List[int]
    step_cows: list
    tables: List[List[int]]
    lens: List[int]
    page_size: int
    mirror: Optional[PoolMirror] = None


def run_single_step(wl, page_size: int = None, with_mirror: bool = True, free_order=None) -> SingleStep:
    P = wl.cfg.page_size if page_size is None else page_size
    hot = HotPool(wl.hot_capacity)
    bases = admit_prefixes(hot, wl)
    fo = wl.free_order if free_order is None else free_order
    cold = ColdPool(wl.num_cold_pages, P, None if fo is None else list(fo))
    B = wl.batch
    seqs = [cold.seq_new() for _ in range(B)]
    setup_ids = [seqs[b] for b in range(B) for _ in range(int(wl.suffix_len[b]) - 1)]
    setup_slots, _, n_done, err = cold.append_batch(setup_ids)
    assert err is None, err
    step_slots, step_cows, n_done, err = cold.append_batch(seqs)
    assert err is None, err
    mirror = None
    if with_mirror:
        hkv, d = wl.cfg.num_kv_heads, wl.cfg.head_dim
        mirror = PoolMirror(wl.hot_capacity, wl.num_cold_pages * P, hkv, d, _np_dtype(wl))
        for g, base in enumerate(bases):
            mirror.hot_write(wl.prefix_k[g], wl.prefix_v[g], base)
        off = wl.suffix_offsets
        setup_rows = np.concatenate([np.arange(off[b], off[b + 1] - 1) for b in range(B)]) if B else np.zeros(0, int)
        mirror.reshape_and_cache(wl.suffix_k[setup_rows], wl.suffix_v[setup_rows], setup_slots)
        mirror.copy_blocks(step_cows, P)
        last_rows = off[1:] - 1
        mirror.reshape_and_cache(wl.suffix_k[last_rows], wl.suffix_v[last_rows], step_slots)
    tables = [cold.block_table(s) for s in seqs]
    lens = [cold.length(s) for s in seqs]
    return SingleStep(hot, cold, bases, seqs, setup_slots, step_slots, step_cows, tables, lens, P, mirror)


def paged_reference(st: SingleStep, wl, scale: float = None):
    """Attention read back through the pool mirror (HOT slab + block tables)."""
    cfg = wl.cfg
    dt, G, hkv = cfg.dtype, cfg.group_size, cfg.num_kv_heads
    scale = (1.0 / np.sqrt(cfg.head_dim)) if scale is None else scale
    B, Hq, d = wl.q.shape
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), NEG_INF)
    for b in range(B):
        g = int(wl.group_of[b])
        parts_k, parts_v = [], []
        if g >= 0:
            pk, pv = st.mirror.gather_prefix(st.bases[g], int(wl.group_prefix_len[g]))
            parts_k.append(widen(pk, dt)); parts_v.append(widen(pv, dt))
        sk, sv = st.mirror.gather_suffix(st.tables[b], st.lens[b], st.page_size)
        parts_k.append(widen(sk, dt)); parts_v.append(widen(sv, dt))
        q = widen(wl.q[b], dt)
        for h in range(hkv):
            r = slice(h * G, (h + 1) * G)
            out[b, r], lse[b, r] = attend(q[r], [p[:, h] for p in parts_k], [p[:, h] for p in parts_v], scale)
    return out, lse


@dataclass
class StepRecord:
    live: List[int]                 # request ids attended this step, ascending
    slots: List[int]
    cows: list
    tables: Dict[int, List[int]]
    lens: Dict[int, int]
    forked: Dict[int, int] = field(default_factory=dict)   # parent -> child at this step
    released: List[int] = field(default_factory=list)


class MultiStepSim:
    """Oracle side of the multi-step run (allocators + logical K/V history)."""

    def __init__(self, wl, page_size: int = None, fork_step: int = 8, release_step: int = 24,
                 keep_history: bool = True):
        self.wl = wl
        self.P = wl.cfg.page_size if page_size is None else page_size
        self.fork_step, self.release_step = fork_step, release_step
        self.hot = HotPool(wl.hot_capacity)
        self.bases = admit_prefixes(self.hot, wl)
        fo = wl.free_order
        self.cold = ColdPool(wl.num_cold_pages, self.P, None if fo is None else list(fo))
        B = wl.batch
        self.group_of: Dict[int, int] = {}
        self.live: List[int] = []
        for b in range(B):
            sid = self.cold.seq_new()
            assert sid == b
            self.group_of[sid] = int(wl.group_of[b])
            self.live.append(sid)
        setup_ids = [b for b in range(B) for _ in range(int(wl.suffix_len[b]) - 1)]
        self.setup_slots, _, n, err = self.cold.append_batch(setup_ids)
        assert err is None, err
        self.keep_history = keep_history
        self.hist_k: Dict[int, list] = {}
        self.hist_v: Dict[int, list] = {}
        if keep_history:
            for b in range(B):
                sk, sv = wl.suffix_kv(b)
                self.hist_k[b] = [sk[:-1]]
                self.hist_v[b] = [sv[:-1]]
        self.fork_parents: List[int] = []
        self.step_index = 0

    def step(self, k_new, v_new) -> StepRecord:
        """Advance one step.  k_new/v_new: [n_live_after_fork_release, Hkv, d] in live order."""
        s = self.step_index
        forked, released = {}, []
        if s == self.fork_step:
            firsts = {}
            for b in sorted(self.live):
                g = self.group_of[b]
                if g >= 0 and g not in firsts:
                    firsts[g] = b
            for g in sorted(firsts):
                parent = firsts[g]
                child = self.cold.fork(parent)
                self.hot.incref(self.bases[g])
                self.group_of[child] = g
                self.live.append(child)
                forked[parent] = child
                self.fork_parents.append(parent)
                if self.keep_history:
                    self.hist_k[child] = list(self.hist_k[parent])
                    self.hist_v[child] = list(self.hist_v[parent])
        if s == self.release_step:
            for parent in sorted(self.fork_parents):
                self.cold.release(parent)
                g = self.group_of[parent]
                if g >= 0:
                    self.hot.decref(self.bases[g])
                self.live.remove(parent)
                released.append(parent)
        live = sorted(self.live)
        slots, cows, n, err = self.cold.append_batch(live)
        assert err is None, err
        if self.keep_history:
            for i, b in enumerate(live):
                self.hist_k[b].append(k_new[i:i + 1])
                self.hist_v[b].append(v_new[i:i + 1])
        tables = {b: self.cold.block_table(b) for b in live}
        lens = {b: self.cold.length(b) for b in live}
        self.step_index += 1
        return StepRecord(live, slots, cows, tables, lens, forked, released)

    def reference(self, live: List[int], q: np.ndarray, rows: List[int] = None, scale: float = None):
        """Flat fp64 reference for this step's live requests (q in live order)."""
        wl = self.wl
        cfg = wl.cfg
        dt, G, hkv = cfg.dtype, cfg.group_size, cfg.num_kv_heads
        scale = (1.0 / np.sqrt(cfg.head_dim)) if scale is None else scale
        n, Hq, d = q.shape
        out = np.zeros((n, Hq, d))
        lse = np.full((n, Hq), NEG_INF)
        pk = {}
        for i in (range(n) if rows is None else rows):
            b = live[i]
            g = self.group_of[b]
            if g >= 0 and g not in pk:
                pk[g] = (widen(wl.prefix_k[g], dt), widen(wl.prefix_v[g], dt))
            sk = widen(np.concatenate(self.hist_k[b], axis=0), dt)
            sv = widen(np.concatenate(self.hist_v[b], axis=0), dt)
            qb = widen(q[i], dt)
            for h in range(hkv):
                r = slice(h * G, (h + 1) * G)
                ks = ([pk[g][0][:, h]] if g >= 0 else []) + [sk[:, h]]
                vs = ([pk[g][1][:, h]] if g >= 0 else []) + [sv[:, h]]
                out[i, r], lse[i, r] = attend(qb[r], ks, vs, scale)
        return out, lse

    def reference_grouped(self, live: List[int], q: np.ndarray, scale: float = None):
        """The same values for every live request, each group's prefix widened
        once and attended by all of its members' rows together."""
        wl = self.wl
        cfg = wl.cfg
        dt, G, hkv = cfg.dtype, cfg.group_size, cfg.num_kv_heads
        scale = (1.0 / np.sqrt(cfg.head_dim)) if scale is None else scale
        n, Hq, d = q.shape
        out = np.zeros((n, Hq, d))
        lse = np.full((n, Hq), NEG_INF)
        by_group: Dict[int, List[int]] = {}
        for i, b in enumerate(live):
            by_group.setdefault(self.group_of[b], []).append(i)
        for g, idx in sorted(by_group.items()):
            pk = widen(wl.prefix_k[g], dt) if g >= 0 else None
            pv = widen(wl.prefix_v[g], dt) if g >= 0 else None
            suffix = [(widen(np.concatenate(self.hist_k[live[i]], axis=0), dt),
                       widen(np.concatenate(self.hist_v[live[i]], axis=0), dt)) for i in idx]
            for h in range(hkv):
                qr = np.concatenate([widen(q[i, h * G:(h + 1) * G], dt) for i in idx])
                parts = [(slice(j * G, (j + 1) * G), sk[:, h], sv[:, h]) for j, (sk, sv) in enumerate(suffix)]
                o, l = attend_shared_prefix(qr, None if pk is None else pk[:, h], None if pv is None else pv[:, h],
                                            parts, scale)
                for j, i in enumerate(idx):
                    out[i, h * G:(h + 1) * G] = o[j * G:(j + 1) * G]
                    lse[i, h * G:(h + 1) * G] = l[j * G:(j + 1) * G]
        return out, lse

    def finish(self) -> int:
        for b in sorted(self.live):
            self.cold.release(b)
            g = self.group_of[b]
            if g >= 0:
                self.hot.decref(self.bases[g])
        self.live = []
        return self.hot.evict_unreferenced()
