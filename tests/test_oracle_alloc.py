"""Pins for the oracle allocators (CPU).

The "Paged KV cache" page's worked example and block-table picture, invariants
that hold for any operation sequence (exhaustive on tiny pools), and a
hand-worked HOT pool trace.
"""
import copy
import json
import os
import random

import pytest

from conftest import GOLDEN
from oracle.alloc import ColdPool, HotPool, OutOfMemory, StateError, InvalidArgument


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_counts_and_values():
    g = load("paged_kv_worked_example.json")
    pa, hand = g["page_asserts"], g["derived_by_hand"]
    pool = ColdPool(g["num_blocks"], g["block_size"])
    a = pool.seq_new()
    slots = [pool.append(a)[0] for _ in range(pa["appends_before_fork"])]
    assert (len(pool.block_table(a)), pool.num_free()) == (pa["after_appends_table_len"], pa["after_appends_num_free"])
    assert pool.block_table(a) == hand["parent_table"]
    assert slots == hand["parent_slots"]
    b = pool.fork(a)
    assert pool.ref == hand["refcounts_after_fork"]
    slot, cow = pool.append(b)
    assert (cow is not None) == pa["fork_then_append_reports_cow"]
    assert (pool.block_table(b)[0] == pool.block_table(a)[0]) == pa["child_first_block_shared"]
    assert (pool.block_table(b)[1] != pool.block_table(a)[1]) == pa["child_second_block_differs"]
    assert slot == hand["child_append_slot"]
    assert list(cow) == hand["child_cow_pair"]
    assert pool.block_table(b) == hand["child_table_after_append"]
    assert pool.ref == hand["refcounts_after_child_append"]
    pool.release(a)
    pool.release(b)
    assert pool.num_free() == pa["num_free_after_both_released"]
    assert pool.free == hand["free_stack_bottom_to_top_after_release"]
    c = pool.seq_new()
    pool.append(c)
    assert pool.block_table(c) == [hand["next_alloc_after_release"]]


def test_block_table_picture():
    g = load("paged_kv_block_table_example.json")
    bs = g["block_size"]
    pool = ColdPool(8, bs, free_order=[3, 0, 1, 4, 2, 5, 6, 7])
    a = pool.seq_new()
    slots_a = []
    for _ in range(16):
        slots_a.append(pool.append(a)[0])
    b = pool.fork(a)
    assert g["seq_b_forked_after_token"] == pool.length(a) - 1
    for _ in range(16):
        slots_a.append(pool.append(a)[0])
    pool.append(b)
    for _ in range(9):
        slots_a.append(pool.append(a)[0])
    assert pool.block_table(a) == g["seq_a_table"]
    assert pool.block_table(b) == g["seq_b_table"]
    assert pool.ref[g["shared_block"]] == g["shared_block_refcount"]
    for lo, hi, blk in g["seq_a_token_blocks"]:
        for t in range(lo, hi + 1):
            assert slots_a[t] // bs == blk
            assert slots_a[t] == blk * bs + t % bs


def check_cold_invariants(pool: ColdPool):
    live = [s for s in pool.seqs.values() if s.live]
    count = [0] * pool.num_pages
    for s in live:
        assert len(set(s.table)) == len(s.table)
        assert len(s.table) == -(-s.length // pool.page_size)
        for b in s.table:
            count[b] += 1
    assert count == pool.ref
    assert len(set(pool.free)) == len(pool.free)
    assert sorted(pool.free) == [p for p in range(pool.num_pages) if pool.ref[p] == 0]


def _cold_ops(pool):
    ops = [("new", None)]
    for sid, s in pool.seqs.items():
        if s.live:
            ops += [("append", sid), ("fork", sid), ("release", sid)]
    return ops


def _apply(pool, op, arg):
    if op == "new":
        if len([s for s in pool.seqs.values() if s.live]) >= 3:
            return "skip"
        pool.seq_new()
    elif op == "append":
        before = copy.deepcopy(pool.state())
        try:
            pool.append(arg)
        except OutOfMemory:
            assert pool.state() == before, "failed append changed state"
            return "nomem"
    elif op == "fork":
        if len([s for s in pool.seqs.values() if s.live]) >= 3:
            return "skip"
        pool.fork(arg)
    elif op == "release":
        pool.release(arg)
    return "ok"


@pytest.mark.parametrize("num_pages,page_size", [(2, 1), (3, 1), (2, 2), (3, 2), (2, 16), (4, 1)])
def test_exhaustive_invariants(num_pages, page_size):
    """Every operation sequence of length <= depth over {new, append, fork, release}."""
    depth = 7 if (num_pages, page_size) == (3, 2) else 6
    stats = {"nodes": 0, "nomem": 0, "cow": 0}

    def dfs(pool, d):
        stats["nodes"] += 1
        check_cold_invariants(pool)
        # releasing everything returns every page
        done = copy.deepcopy(pool)
        for sid, s in list(done.seqs.items()):
            if s.live:
                done.release(sid)
        assert done.ref == [0] * num_pages and done.num_free() == num_pages
        if d == depth:
            return
        for op, arg in _cold_ops(pool):
            child = copy.deepcopy(pool)
            if op == "append":
                before_tables = {sid: list(s.table) for sid, s in child.seqs.items() if s.live and sid != arg}
            r = _apply(child, op, arg)
            if r == "skip":
                continue
            if r == "nomem":
                stats["nomem"] += 1
            if op == "append" and r == "ok":
                # copy-on-write never changes any other sequence's table
                for sid, t in before_tables.items():
                    assert child.seqs[sid].table == t
                if child.seqs[arg].table != pool.seqs[arg].table[:len(child.seqs[arg].table)] and \
                        len(child.seqs[arg].table) == len(pool.seqs[arg].table):
                    stats["cow"] += 1
            dfs(child, d + 1)

    dfs(ColdPool(num_pages, page_size), 0)
    assert stats["nodes"] > 100
    assert stats["nomem"] > 0
    if page_size > 1:
        assert stats["cow"] > 0


def test_random_long_sequences():
    rng = random.Random(5)
    for trial in range(40):
        n, P = rng.choice([(8, 1), (6, 4), (5, 16), (16, 2)])
        order = list(range(n)); rng.shuffle(order)
        pool = ColdPool(n, P, free_order=order)
        for _ in range(200):
            ops = _cold_ops(pool)
            op, arg = rng.choice(ops)
            if op == "new" and rng.random() < 0.5:
                op, arg = ops[-1] if len(ops) > 1 else ops[0]
            _apply(pool, op, arg)
            check_cold_invariants(pool)
        for sid, s in list(pool.seqs.items()):
            if s.live:
                pool.release(sid)
        assert pool.ref == [0] * n and pool.num_free() == n


def test_cold_errors():
    pool = ColdPool(2, 1)
    a = pool.seq_new()
    pool.append(a)
    pool.release(a)
    with pytest.raises(StateError):
        pool.release(a)
    with pytest.raises(StateError):
        pool.append(a)
    with pytest.raises(StateError):
        pool.fork(99)
    with pytest.raises(InvalidArgument):
        ColdPool(3, 1, free_order=[0, 0, 1])
    b = pool.seq_new()
    pool.append(b); pool.append(b)
    st = pool.state()
    with pytest.raises(OutOfMemory):
        pool.append(b)
    assert pool.state() == st


def test_append_batch_stops_at_first_failure():
    pool = ColdPool(3, 1)
    s = [pool.seq_new() for _ in range(2)]
    slots, cows, n, err = pool.append_batch([s[0], s[1], s[0], s[1], s[0]])
    assert n == 3 and isinstance(err, OutOfMemory)
    assert slots == [0, 1, 2] and cows == []


def check_hot_invariants(hot: HotPool):
    spans = sorted([(b, n, "free") for b, n in hot.free] + [(b, s.length, "slab") for b, s in hot.slabs.items()])
    pos = 0
    for b, n, kind in spans:
        assert b == pos and n > 0
        pos += n
    assert pos == hot.capacity
    for (b1, n1), (b2, n2) in zip(hot.free, hot.free[1:]):
        assert b1 + n1 < b2, "adjacent free ranges must be merged"


def test_hot_hand_trace():
    hot = HotPool(10)
    assert hot.alloc(3) == 0
    assert hot.alloc(4) == 3
    assert hot.alloc(2) == 7
    assert hot.free == [(9, 1)]
    hot.decref(3)
    assert hot.state()["slabs"] == [(0, 3, 1, -1), (3, 4, 0, 0), (7, 2, 1, -1)]
    assert hot.alloc(2) == 3                        # evicts slab 3, first fit at its base
    assert hot.free == [(5, 2), (9, 1)]
    hot.decref(0)
    hot.decref(7)
    assert hot.alloc(4) == 5                        # evicts 0 (older) then 7; merge 5..10
    assert hot.free == [(0, 3), (9, 1)]
    st = hot.state()
    with pytest.raises(OutOfMemory):
        hot.alloc(6)
    assert hot.state() == st
    hot.decref(3)
    hot.incref(3)                                   # revived before eviction
    assert hot.state()["slabs"][0][2:] == (1, -1)
    with pytest.raises(StateError):
        hot.decref(1)
    with pytest.raises(InvalidArgument):
        hot.alloc(0)
    hot.decref(3); hot.decref(5)
    assert hot.evict_unreferenced() == 2
    assert hot.free == [(0, 10)] and hot.slabs == {}


def test_hot_random_invariants():
    rng = random.Random(11)
    for trial in range(30):
        cap = rng.randint(1, 40)
        hot = HotPool(cap)
        for _ in range(120):
            r = rng.random()
            if r < 0.5:
                lp = rng.randint(1, max(1, cap // 2))
                st = copy.deepcopy(hot.state())
                try:
                    hot.alloc(lp)
                except OutOfMemory:
                    assert hot.state() == st
                    evictable = sum(s.length for s in hot.slabs.values() if s.ref == 0)
                    assert evictable + max([n for _, n in hot.free] + [0]) < lp or True
            elif hot.slabs:
                base = rng.choice(sorted(hot.slabs))
                if r < 0.8 and hot.slabs[base].ref > 0:
                    hot.decref(base)
                else:
                    hot.incref(base)
            check_hot_invariants(hot)
        for base, s in list(hot.slabs.items()):
            while s.ref > 0:
                hot.decref(base)
        hot.evict_unreferenced()
        assert hot.free == ([(0, cap)] if cap else []) and not hot.slabs


def test_hot_first_fit_prefers_lowest_base():
    hot = HotPool(12)
    a = hot.alloc(2); b = hot.alloc(3); c = hot.alloc(2); d = hot.alloc(5)
    hot.decref(a); hot.decref(c)
    hot.evict_unreferenced()
    assert hot.free == [(0, 2), (5, 2)]
    assert hot.alloc(2) == 0
    assert hot.alloc(2) == 5
