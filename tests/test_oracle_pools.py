"""Pins for the oracle's pool mirror (CPU): addressing, reshape_and_cache,
copy_blocks and the copy-on-write invariant.

Each test names the mistake it catches.
"""
import hashlib
import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle.alloc import ColdPool, HotPool
from oracle.pools import PoolMirror, cold_slot, hot_offset


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def token_rows(n, hkv, d, start=1):
    """Token i's K row is filled with the value start + i (exact in float32)."""
    return np.repeat(np.arange(start, start + n, dtype=np.float32), hkv * d).reshape(n, hkv, d)


def test_hot_offset_hand_value():
    # "GraniKV" paper, Section 3.2: head h of a slab at token slot `base` starts
    # at row base*Hkv + h*Lp.  base 3, Lp 5, Hkv 2, d 4, token 2 of head 1:
    # rows 3*2 = 6 (slab start) + 1*5 (head 1) + 2 = 13, element 13*4 = 52.
    # Catches: a token-major slab (would give (3*2 + 2*2 + 1)*4 = 44) or a
    # missing Hkv factor on the base (would be (3 + 5 + 2)*4 = 40).
    assert hot_offset(3, 5, 2, 4, 2, 1) == 52
    assert hot_offset(0, 7, 3, 8, 0, 0) == 0
    assert hot_offset(0, 7, 3, 8, 6, 2) == (2 * 7 + 6) * 8


def test_hot_write_places_heads_as_dense_matrices():
    # Catches: heads interleaved per token instead of one dense [Lp, d] block per head.
    hkv, d, lp, base = 2, 4, 3, 1
    m = PoolMirror(hot_capacity=5, cold_slots=0, hkv=hkv, d=d, np_dtype=np.float32)
    k = np.arange(lp * hkv * d, dtype=np.float32).reshape(lp, hkv, d)
    m.hot_write(k, -k, base)
    # Head 0's rows of the slab: rows base*Hkv + 0 .. +2 = 2, 3, 4; head 1: 5, 6, 7.
    rows = m.k_hot.reshape(-1, d)
    np.testing.assert_array_equal(rows[2:5], k[:, 0])
    np.testing.assert_array_equal(rows[5:8], k[:, 1])
    assert not rows[:2].any() and not rows[8:].any()      # nothing outside the slab
    pk, pv = m.gather_prefix(base, lp)
    np.testing.assert_array_equal(pk, k)
    np.testing.assert_array_equal(pv, -k)


def test_block_table_picture_through_the_mirror():
    # "Paged KV cache" page, How it works: tokens 0-15 in block 3, 16-31 in
    # block 0, 32-40 in block 4 (block size 16).  Tokens written at their
    # slots land in those blocks and read back in logical order.
    # Catches: slot = table[t % P] * P + t // P (swapped div/mod), or an
    # off-by-one page for token 16 / 32.
    g = load("paged_kv_block_table_example.json")
    P = g["block_size"]
    pool = ColdPool(8, P, free_order=[3, 0, 1, 4, 2, 5, 6, 7])
    a = pool.seq_new()
    # The picture's history: A's first 16 tokens, B forks, A's next 16, B's
    # one token of its own, A's last 9.
    slots = [pool.append(a)[0] for _ in range(16)]
    b = pool.fork(a)
    slots += [pool.append(a)[0] for _ in range(16)]
    pool.append(b)
    slots += [pool.append(a)[0] for _ in range(9)]
    assert pool.block_table(a) == g["seq_a_table"] and pool.block_table(b) == g["seq_b_table"]
    assert pool.ref[g["shared_block"]] == g["shared_block_refcount"]
    for lo, hi, blk in g["seq_a_token_blocks"]:
        for t in range(lo, hi + 1):
            assert slots[t] // P == blk and slots[t] % P == t % P
            assert cold_slot(pool.block_table(a), t, P) == slots[t]
    hkv, d = 1, 2
    m = PoolMirror(0, 8 * P, hkv, d, np.float32)
    k = token_rows(41, hkv, d)
    m.reshape_and_cache(k, -k, slots)
    # block 3 holds tokens 0..15 in row order, block 0 tokens 16..31, block 4 tokens 32..40
    np.testing.assert_array_equal(m.k_cold.reshape(-1, d)[3 * P:4 * P, 0], np.arange(1, 17))
    np.testing.assert_array_equal(m.k_cold.reshape(-1, d)[0:P, 0], np.arange(17, 33))
    np.testing.assert_array_equal(m.k_cold.reshape(-1, d)[4 * P:4 * P + 9, 0], np.arange(33, 42))
    gk, gv = m.gather_suffix(pool.block_table(a), 41, P)
    np.testing.assert_array_equal(gk, k)
    np.testing.assert_array_equal(gv, -k)


def test_reshape_and_cache_skips_slots_outside_the_pool():
    # Catches: a negative slot wrapping around to the end of the pool (numpy
    # negative indexing) instead of being skipped.
    m = PoolMirror(0, 3, 1, 2, np.float32)
    k = token_rows(3, 1, 2)
    m.reshape_and_cache(k, k, [2, -1, 3])
    np.testing.assert_array_equal(m.k_cold.reshape(3, 2), [[0, 0], [0, 0], [1, 1]])


def test_copy_blocks_hand_worked_two_pages():
    # Page size 2, one KV head of d = 2: a page is 2 rows x 2 values.
    # Before: page 0 = [[1,1],[2,2]], page 1 = [[3,3],[4,4]], page 2 = 0.
    # copy_blocks([(0, 2)]) makes page 2 = [[1,1],[2,2]] and leaves pages 0, 1.
    # Catches: copying one row instead of the page (P*Hkv*d values), copying
    # dst -> src, or touching any other page.
    m = PoolMirror(0, 6, 1, 2, np.float32)
    m.reshape_and_cache(token_rows(4, 1, 2), -token_rows(4, 1, 2), [0, 1, 2, 3])
    m.copy_blocks([(0, 2)], page_size=2)
    np.testing.assert_array_equal(m.k_cold.reshape(3, 2, 2),
                                  [[[1, 1], [2, 2]], [[3, 3], [4, 4]], [[1, 1], [2, 2]]])
    np.testing.assert_array_equal(m.v_cold.reshape(3, 2, 2),
                                  -np.array([[[1, 1], [2, 2]], [[3, 3], [4, 4]], [[1, 1], [2, 2]]]))
    # Pairs apply in order: (1, 0) then (0, 2) copies page 1 through page 0 into page 2.
    # Catches: applying the pairs in reverse or all from a snapshot.
    m.copy_blocks([(1, 0), (0, 2)], page_size=2)
    np.testing.assert_array_equal(m.k_cold.reshape(3, 2, 2),
                                  [[[3, 3], [4, 4]], [[3, 3], [4, 4]], [[3, 3], [4, 4]]])


def test_copy_blocks_with_two_heads_copies_every_head():
    # Catches: a page span of P*d (one head) instead of P*Hkv*d.
    hkv, d, P = 2, 3, 2
    m = PoolMirror(0, 3 * P, hkv, d, np.float32)
    k = np.arange(2 * hkv * d, dtype=np.float32).reshape(2, hkv, d) + 1
    m.reshape_and_cache(k, k, [2, 3])          # page 1
    m.copy_blocks([(1, 0)], page_size=P)
    np.testing.assert_array_equal(m.k_cold.reshape(3, P, hkv, d)[0], k)
    np.testing.assert_array_equal(m.k_cold.reshape(3, P, hkv, d)[1], k)


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("fork_at", [20, 32, 33])
def test_copy_on_write_leaves_shared_pages_and_slab_untouched(fork_at):
    # North-star invariant (P4), "Paged KV cache" page, Code (fork shares
    # pages; a write to a shared page goes to a private copy): at P = 16, a
    # parent with a HOT prefix and `fork_at` suffix tokens forks; parent and
    # child each append a token (the step's appends in ascending id, the
    # copy-on-write copies, then the writes).  Every row that held a token
    # before the fork, on every page the parent held, and the whole HOT slab
    # are byte-identical afterwards.
    # Catches: writing a token into a page that is still shared (no CoW), a
    # CoW copy in the wrong direction (dst -> src overwrites the shared rows),
    # or a copy that spills into the slab.
    P, hkv, d, lp = 16, 2, 4, 24
    rng = np.random.default_rng(fork_at)
    hot = HotPool(lp)
    base = hot.alloc(lp)
    pool = ColdPool(12, P, free_order=list(rng.permutation(12)))
    m = PoolMirror(lp, 12 * P, hkv, d, np.float32)
    pk = rng.standard_normal((lp, hkv, d)).astype(np.float32)
    m.hot_write(pk, -pk, base)
    parent = pool.seq_new()
    hist = rng.standard_normal((fork_at, hkv, d)).astype(np.float32)
    slots = [pool.append(parent)[0] for _ in range(fork_at)]
    m.reshape_and_cache(hist, -hist, slots)
    table0 = list(pool.block_table(parent))

    def shared_rows():
        k, v = m.gather_suffix(table0, fork_at, P)       # the pre-fork rows, at their pre-fork slots
        return digest(k, v, m.k_hot, m.v_hot)

    before = shared_rows()
    child = pool.fork(parent)
    hot.incref(base)
    new = rng.standard_normal((2, hkv, d)).astype(np.float32)
    step_slots, cows, n, err = pool.append_batch([parent, child])
    assert err is None and n == 2
    m.copy_blocks(cows, P)
    m.reshape_and_cache(new, -new, step_slots)
    assert shared_rows() == before

    # Only a partially filled shared page needs a copy: the parent appends
    # first, takes a private copy, and the old page is left to the child.
    if fork_at % P:
        (src, dst), = cows
        assert src == table0[-1] and pool.block_table(parent) == table0[:-1] + [dst]
        assert pool.block_table(child) == table0
    else:
        assert cows == [] and pool.block_table(parent)[:-1] == pool.block_table(child)[:-1] == table0
    assert not set(step_slots) & set(slots)              # no new token overwrote a pre-fork row
    # Both sequences read back the shared history plus their own token.
    for sid, tok in ((parent, new[0]), (child, new[1])):
        gk, gv = m.gather_suffix(pool.block_table(sid), fork_at + 1, P)
        np.testing.assert_array_equal(gk[:fork_at], hist)
        np.testing.assert_array_equal(gk[fork_at], tok)
        np.testing.assert_array_equal(gv[fork_at], -tok)
    pk2, pv2 = m.gather_prefix(base, lp)
    np.testing.assert_array_equal(pk2, pk)
    np.testing.assert_array_equal(pv2, -pk)


def test_copy_on_write_check_fails_without_the_copy():
    # The P4 check above must be able to fail: skipping copy-on-write (both
    # sequences write into the shared partial page) puts the child's token on
    # the parent's row.  Planted here, on the CPU, in a copy of the logic.
    P, hkv, d = 16, 1, 2
    pool = ColdPool(4, P)
    m = PoolMirror(0, 4 * P, hkv, d, np.float32)
    a = pool.seq_new()
    hist = token_rows(20, hkv, d)
    m.reshape_and_cache(hist, hist, [pool.append(a)[0] for _ in range(20)])
    b = pool.fork(a)
    # a CoW-less append: both tokens go to row 4 of the shared second page
    shared_slot = pool.block_table(a)[1] * P + 20 % P
    m.reshape_and_cache(token_rows(2, hkv, d, start=100), token_rows(2, hkv, d, start=100),
                        [shared_slot, shared_slot])
    ka, _ = m.gather_suffix(pool.block_table(a), 21, P)
    assert ka[20, 0, 0] == 101.0                         # the parent now reads the child's token


def test_layer_stride_hand_values():
    # GraniKV paper, Section 3.2: head h of layer l sits at base + l*Lp*Hkv + h*Lp
    # (rows) inside the prefix's slab, which starts at row base*Hkv*L.  base 2,
    # Lp 5, Hkv 3, L 4, layer 2, head 1, token 4, d 8:
    # slab start 2*3*4 = 24, layer 2*5*3 = 30, head 1*5 = 5, token 4 -> row 63.
    # Catches: a layer term of l*Lp (missing Hkv), a slab start without L, or
    # layers interleaved per head (h*Lp*L + l*Lp).
    assert hot_offset(2, 5, 3, 8, 4, 1, layer=2, num_layers=4) == 63 * 8
    assert hot_offset(2, 5, 3, 8, 4, 1) == (2 * 3 + 5 + 4) * 8          # one layer: the single-layer formula
    # Consecutive layers of one head are Lp*Hkv rows apart; the next slab
    # (base + Lp) starts right after the last layer of this one.
    assert hot_offset(0, 5, 3, 8, 0, 0, 1, 4) - hot_offset(0, 5, 3, 8, 0, 0, 0, 4) == 5 * 3 * 8
    assert hot_offset(5, 7, 3, 8, 0, 0, 0, 4) == hot_offset(0, 5, 3, 8, 4, 2, 3, 4) + 8


def test_multi_layer_pools_keep_layers_apart_and_copy_pages_in_every_layer():
    # Two layers sharing slots: layer 1's writes never touch layer 0, a prefix
    # written per layer reads back per layer, and a copy-on-write pair copies
    # the page in both layers.  Catches: a COLD layer offset of 0, or
    # copy_blocks copying only the first layer.
    hkv, d, P, L = 2, 2, 2, 2
    m = PoolMirror(hot_capacity=6, cold_slots=8, hkv=hkv, d=d, np_dtype=np.float32, num_layers=L)
    pk = [np.arange(3 * hkv * d, dtype=np.float32).reshape(3, hkv, d) + 100 * (l + 1) for l in range(L)]
    for l in range(L):
        m.hot_write(pk[l], -pk[l], base=2, layer=l)
    for l in range(L):
        k, v = m.gather_prefix(2, 3, layer=l)
        np.testing.assert_array_equal(k, pk[l])
        np.testing.assert_array_equal(v, -pk[l])
    rows = [token_rows(2, hkv, d, start=1 + 10 * l) for l in range(L)]
    for l in range(L):
        m.reshape_and_cache(rows[l], rows[l], [2, 3], layer=l)        # page 1 in both layers
    m.copy_blocks([(1, 3)], page_size=P)
    for l in range(L):
        k, _ = m.gather_suffix([3], 2, P, layer=l)
        np.testing.assert_array_equal(k, rows[l])
        k, _ = m.gather_suffix([1], 2, P, layer=l)
        np.testing.assert_array_equal(k, rows[l])
    assert not m.k_cold[:P * hkv * d].any()                            # layer 0's page 0 untouched
