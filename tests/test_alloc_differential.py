"""The native allocators (libspkv.so, host code, no GPU needed) against the
oracle allocators: identical slots, copy-on-write pairs, tables, refcounts,
free stacks, HOT ranges and errors, operation by operation (CPU only)."""
import random

import pytest

import shared_prefix_paged_amd as spkv
from shared_prefix_paged_amd.runtime import ColdPool as NativeCold, HotPool as NativeHot
from oracle import alloc as O


def cold_ops(oracle: O.ColdPool, max_live=4):
    live = [sid for sid, s in oracle.seqs.items() if s.live]
    ops = []
    if len(live) < max_live:
        ops.append(("new", None))
    for sid in live:
        ops += [("append", sid), ("release", sid)]
        if len(live) < max_live:
            ops.append(("fork", sid))
    ops.append(("append", 10_000))   # unknown id -> state error on both sides
    return ops


def apply_both(o: O.ColdPool, n: NativeCold, op, arg):
    if op == "new":
        assert o.seq_new() == n.seq_new()
    elif op == "append":
        try:
            ro = o.append(arg)
            eo = None
        except O.PoolError as e:
            ro, eo = None, e
        st, slots, pairs, done = n.append_batch_raw([arg])
        if eo is None:
            assert st == 0 and done == 1
            assert int(slots[0]) == ro[0]
            assert (pairs[0] if pairs else None) == ro[1]
        else:
            assert st == eo.code and done == 0
    elif op == "fork":
        assert o.fork(arg) == n.fork(arg)
    elif op == "release":
        o.release(arg)
        n.release(arg)


@pytest.mark.parametrize("seed", range(12))
def test_cold_random_sequences(seed):
    rng = random.Random(seed)
    num_pages = rng.choice([3, 5, 8, 13])
    P = rng.choice([1, 2, 4, 16])
    order = list(range(num_pages))
    if rng.random() < 0.7:
        rng.shuffle(order)
    o = O.ColdPool(num_pages, P, order)
    n = NativeCold(num_pages, P, order)
    for step in range(300):
        op, arg = rng.choice(cold_ops(o))
        if op == "append" and rng.random() < 0.5 and arg != 10_000:
            pass
        apply_both(o, n, op, arg)
        assert n.state() == o.state(), f"diverged at step {step} ({op} {arg})"


def test_cold_batch_append_matches_loop():
    rng = random.Random(3)
    for trial in range(20):
        order = list(range(24)); rng.shuffle(order)
        P = rng.choice([1, 4, 16])
        o = O.ColdPool(24, P, order)
        n = NativeCold(24, P, order)
        ids = [o.seq_new() for _ in range(4)]
        assert [n.seq_new() for _ in range(4)] == ids
        for _ in range(6):
            if rng.random() < 0.3:
                src = rng.choice([s for s in o.seqs if o.seqs[s].live])
                assert o.fork(src) == n.fork(src)
            live = [s for s in o.seqs if o.seqs[s].live]
            batch = [rng.choice(live) for _ in range(rng.randint(1, 30))]
            so, co, no, eo = o.append_batch(batch)
            st, sn, cn, nn = n.append_batch_raw(batch)
            assert (nn, list(map(int, sn)), cn) == (no, so, co)
            assert st == (0 if eo is None else eo.code)
            assert n.state() == o.state()


def test_cold_worked_example_native():
    n = NativeCold(8, 16)
    a = n.seq_new()
    slots, _ = n.append_batch([a] * 20)
    assert list(slots) == list(range(20)) and n.num_free() == 6
    b = n.fork(a)
    slot, cow = n.append(b)
    assert (slot, cow) == (36, (1, 2))
    n.release(a); n.release(b)
    assert n.state()["free"] == [7, 6, 5, 4, 3, 1, 0, 2]


@pytest.mark.parametrize("seed", range(10))
def test_hot_random_sequences(seed):
    rng = random.Random(100 + seed)
    cap = rng.choice([1, 7, 32, 100])
    o = O.HotPool(cap)
    n = NativeHot(cap)
    for step in range(300):
        r = rng.random()
        if r < 0.45:
            lp = rng.randint(0, max(1, cap // 2 + 1))
            try:
                bo, eo = o.alloc(lp), None
            except O.PoolError as e:
                bo, eo = None, e
            if eo is None:
                assert n.alloc(lp) == bo
            else:
                with pytest.raises(spkv.SpkvError) as ei:
                    n.alloc(lp)
                assert ei.value.status == eo.code
        elif r < 0.9 and o.slabs:
            base = rng.choice(sorted(o.slabs))
            if rng.random() < 0.6:
                try:
                    o.decref(base); eo = None
                except O.PoolError as e:
                    eo = e
                if eo is None:
                    n.decref(base)
                else:
                    with pytest.raises(spkv.StateError):
                        n.decref(base)
            else:
                o.incref(base); n.incref(base)
        elif r < 0.95:
            assert o.evict_unreferenced() == n.evict_unreferenced()
        else:
            with pytest.raises(spkv.StateError):
                n.incref(cap + 5)
        assert n.state() == o.state(), f"diverged at step {step}"
