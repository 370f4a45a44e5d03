"""Host planning of the paged pass (CPU only): the per-request partial-state
counts reported by spkv_plan_parts equal those of the stream-K definition -
a sub-batch's tokens, concatenated in request order with `head` virtual
tokens (owned by no request) before each non-empty request, cut into
`blocks` equal ranges [floor(k*T/n), floor((k+1)*T/n)), one partial per
(range, request) overlap of real tokens - recomputed here by brute force over
token indices."""
import numpy as np
import pytest
import torch

from shared_prefix_paged_amd import runtime as R


def batch_of(lens, groups, group_len, hkv=8, hq=32, d=128, page=1):
    B = len(lens)
    q = torch.zeros((B, hq, d), dtype=torch.bfloat16)
    mb = max(1, max((l + page - 1) // page for l in lens)) if B else 1
    tables = np.full((B, mb), -1, np.int32)
    bases = list(np.cumsum([0] + list(group_len))[:-1])
    return R.DecodeBatch(q, groups, bases, group_len, tables, lens, page, hkv)


def brute_force_parts(L, nb, head=0):
    """Partial count per request when the virtual token sequence (head
    unowned tokens, then the request's own, for each non-empty request) is cut
    into nb equal ranges."""
    owner = [np.concatenate([np.full(head, -1), np.full(l, r)]) for r, l in enumerate(L) if l > 0]
    owner = np.concatenate(owner).astype(np.int64) if owner else np.zeros(0, np.int64)
    T = len(owner)
    parts = np.zeros(len(L), np.int64)
    for k in range(nb):
        lo, hi = (T * k) // nb, (T * (k + 1)) // nb
        for r in np.unique(owner[lo:hi]):
            if r >= 0:
                parts[r] += 1
    return parts


def test_brute_force_without_head_is_plain_stream_k():
    # head = 0: equal ranges over the real tokens; a request of 10 tokens over
    # ranges of 4 spans 3 or 4 of them depending on where it starts
    assert list(brute_force_parts([10, 6], 4)) == [3, 2]
    # head = 2: virtual sequence [-,-,0x10,-,-,1x6] of 20 cut into 4 ranges of 5
    assert list(brute_force_parts([10, 6], 4, head=2)) == [3, 2]
    # an empty request gets no head and no partial
    assert list(brute_force_parts([3, 0, 3], 2, head=3)) == [1, 0, 1]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_flat_parts_match_equal_range_definition(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(3, 40))
    lens = [int(x) for x in rng.integers(0, 3000, size=B)]
    lens[0] = max(lens[0], 1)
    groups = [int(g) for g in rng.integers(-1, 3, size=B)]
    group_len = [int(x) for x in rng.integers(0, 5000, size=3)]
    bt = batch_of(lens, groups, group_len)
    for cascade in ([1, 1, 1], [0, 0, 0], [1, 0, 1]):
        info = bt.plan(cascade)
        flat, pre = bt.plan_parts(cascade)
        # tokens of the paged pass: COLD, plus the HOT prefix of members of non-cascade groups
        L = np.array([lens[b] + (group_len[groups[b]] if groups[b] >= 0 and not cascade[groups[b]] else 0)
                      for b in range(B)], np.int64)
        head_groups = -(-8 // 4)
        nb = int(info.flat_items) // head_groups
        assert nb >= 1
        assert info.flat_head_tokens >= 0
        np.testing.assert_array_equal(flat, brute_force_parts(L, nb, info.flat_head_tokens))
        assert flat.max() <= info.flat_splits <= info.flat_split_cap
        for b in range(B):
            g = groups[b]
            if g >= 0 and cascade[g] and group_len[g] > 0:
                assert 1 <= pre[b] <= info.prefix_splits
            else:
                assert pre[b] == 0


def test_members_of_one_group_share_prefix_parts():
    bt = batch_of([100, 5, 900, 1], [0, 0, 1, 0], [4096, 300])
    flat, pre = bt.plan_parts(None)
    assert pre[0] == pre[1] == pre[3] >= 1 and pre[2] >= 1
    assert (flat >= 1).all()


@pytest.mark.parametrize("members", [1, 2, 3, 5, 17, 40])
def test_prefix_tile_is_a_built_variant(members):
    # 4 query heads per KV head: members * 4 rows per group; tiles of 1, 2 or 4 waves exist
    bt = batch_of([50] * members, [0] * members, [2048], hkv=8, hq=32)
    info = bt.plan(None)
    assert info.prefix_waves in (1, 2, 4) and info.prefix_key_halves == (2 if info.prefix_waves == 4 else 1)
    assert info.prefix_waves * 32 * info.prefix_mtiles >= members * 4


def test_ragged_parity_cases_take_two_key_halves():
    # the GPU parity cases built for the two-key-half prefix tiles do reach them
    for lens, groups, glen, hq, hkv, d in [
            (list(range(1, 25)), [0] * 18 + [1, 1, 2, 2, -1, 1], [276, 326, 21], 16, 4, 128),
            ([3, 70, 1, 5, 9, 130, 2, 33, 64, 17, 8], [0] * 9 + [1, 1], [545, 7], 8, 1, 64)]:
        info = batch_of(lens, groups, glen, hkv=hkv, hq=hq, d=d).plan(None)
        assert info.prefix_waves == 4 and info.prefix_key_halves == 2
        # the base chunk leaves a ragged last chunk in the longest prefix
        assert max(glen) % info.prefix_chunk != 0


@pytest.mark.parametrize("shape", [
    # (requests, groups, prefix lengths, Hq, Hkv)
    (64, 1, [16384], 32, 8),                 # Llama-3.1-8B layer, one shared prefix
    (128, 1, [16384], 20, 4),                # Qwen-2.5-14B half-head share
    (256, 1, [16384], 10, 2),                # Qwen-2.5-32B quarter-head share
    (256, 1, [4096], 10, 2),
    (256, 1, [32768], 10, 2),
    (128, 8, [2048, 16384, 9000, 4100, 12000, 7000, 15000, 3000], 32, 8),   # eight prefix groups
])
def test_prefix_blocks_fit_one_resident_round(shape):
    # 128 KB of LDS rings per CU (256 CUs) hold two blocks of one key half or
    # one block of two: a grid past that many live blocks runs a second,
    # mostly idle round.
    n, ng, lps, hq, hkv = shape
    groups = [min(i // (n // ng), ng - 1) for i in range(n)]
    bt = batch_of([300] * n, groups, lps, hkv=hkv, hq=hq)
    info = bt.plan(None)
    resident = 2 * 256 // info.prefix_key_halves
    assert 0 < info.prefix_items <= resident
    # and the chunk does not grow past what one round needs
    units = sum(hkv * -(-(groups.count(g) * (hq // hkv)) // (32 * info.prefix_waves)) for g in range(ng))
    assert info.prefix_items >= min(resident, units) // 2


def test_single_launch_only_where_both_plans_keep_their_shapes():
    # The paged pass and the prefix contraction share one launch only where a
    # paged block (4 KV-head waves, d = 128) and a prefix block (4 row waves,
    # two key halves) fill a CU as the two plans count them: one paged
    # sub-batch, bf16, Hkv of 1, 2 or >= 4, a group with more than 32 query
    # rows and a prefix of at least 256 keys.
    def single(lens, groups, group_len, cascade=None, **kw):
        return int(batch_of(lens, groups, group_len, **kw).plan(cascade).single_launch)

    lens = [300] * 64
    assert single(lens, [0] * 64, [16384]) == 1                       # 8B shape, Lp 16K
    assert single(lens, [0] * 64, [16384], cascade=[0]) == 0          # no prefix contraction
    assert single(lens, [0] * 64, [16384], hkv=2, hq=8) == 1          # 2 KV heads: two paged blocks side by side
    assert single(lens, [0] * 64, [16384], hkv=1, hq=4) == 1          # 1 KV head: four
    assert single(lens, [0] * 64, [16384], hkv=3, hq=12) == 0         # 3 KV heads: blocks of 3 waves
    assert single(lens, [0] * 64, [16384], d=64) == 0                 # d = 64: two paged blocks per CU
    assert single(lens, [0] * 64, [200]) == 0                         # short prefix: P as hi + lo
    assert single(lens[:8], [0] * 8, [16384]) == 0                    # 32 query rows: tiles of 1 wave
    assert single(lens[:16], [0] * 16, [16384]) == 1                  # 64 query rows: tiles of 2 waves
    assert single(lens[:20], [0] * 20, [16384]) == 1                  # 80 query rows: tiles of 4 waves
    # 2-wave tiles take two key halves only with the one launch (alone, one half per block was faster)
    assert int(batch_of(lens[:16], [0] * 16, [16384]).plan().prefix_key_halves) == 2
    assert int(batch_of(lens[:16], [0] * 16, [16384], d=64).plan().prefix_key_halves) == 1
    assert int(batch_of(lens[:16], [0] * 16, [16384], hkv=3, hq=12).plan().prefix_key_halves) == 1
    assert single([30] * 300, [0] * 300, [16384]) == 0                # two paged sub-batches
    q32 = torch.zeros((64, 32, 128), dtype=torch.float32)
    tables = np.full((64, 300), -1, np.int32)
    assert int(R.DecodeBatch(q32, [0] * 64, [0], [16384], tables, lens, 1, 8).plan().single_launch) == 0


def test_co_resident_where_the_prefix_items_fit_beside_the_paged_blocks():
    # The default one launch runs both roles in every launch block where the
    # prefix items of cascade groups with a prefix, each counted at the plan's
    # row tiles, number no more than the paged blocks: brute-force count here.
    def chunk_for(lp, tau, cap, gran):
        c = max(tau, -(-lp // cap))
        return -(-c // gran) * gran

    def check(lens, groups, group_len, expect, **kw):
        bt = batch_of(lens, groups, group_len, **kw)
        info = bt.plan()
        hkv = kw.get("hkv", 8)
        items = sum(hkv * int(info.prefix_mtiles) * -(-lp // chunk_for(lp, int(info.prefix_chunk), 64, 32))
                    for lp in group_len if lp > 0)
        per = 4 // min(hkv, 4)
        paged = -(-int(info.flat_items) // per)
        assert int(info.co_resident) == int(bool(info.single_launch) and items <= paged) == expect

    check([300] * 64, [0] * 64, [16384], 1)                          # 8B shape, Lp 16K
    # two paged blocks per launch block: 150 launch blocks for 300 ranges, fewer than 256 prefix items
    check([300] * 64, [0] * 64, [16384], 0, hkv=2, hq=8)
    check([300] * 64, [0] * 64, [200], 0)                            # not a single launch at all
    # one large group and seven single-request groups: every group at the large one's row tiles
    check([50] * 107, [0] * 100 + list(range(1, 8)), [2000, 1800, 2100, 1900, 2200, 1700, 2300, 1600], 0)
    # eight groups of 16 (C4 shape): 248 real items in a 6-split x 64 grid, all beside 256 paged blocks
    rng = np.random.default_rng(3)
    lens = [int(x) for x in rng.integers(128, 4096, 128)]
    check(lens, [g for g in range(8) for _ in range(16)], [12134, 14070, 6942, 11971, 5849, 5146, 4709, 3846], 1)


def test_co_resident_ring_depths():
    # The co-resident launch deepens the prefix ring (5 tiles beside paged
    # rings of 2 stages) where a prefix item's key tiles outnumber the 16-token
    # ring stages of a paged wave's range, for tiles of 4 row waves; else 3
    # and 3.  The configurations' shapes, with the counts recomputed here.
    rng = np.random.default_rng(5)

    def check(lens, groups, group_len, expect, **kw):
        info = batch_of(lens, groups, group_len, **kw).plan()
        assert int(info.co_resident) == 1
        lp = max(group_len)
        chunk = max(int(info.prefix_chunk), -(-lp // 64))
        chunk = -(-chunk // 32) * 32
        tiles = -(-min(lp, chunk) // 32)
        stages = -(-int(info.flat_chunk) // 16)
        deep = int(info.prefix_waves) == 4 and tiles > stages
        assert int(info.co_prefix_stages) == (5 if deep else 3) == expect

    # 8B shape, 64 requests, Lp 16K: 32 tiles per item, ~44 stages per paged range
    check([int(x) for x in rng.integers(256, 2049, 64)], [0] * 64, [16384], 3)
    # 32B-shaped share, 256 requests: 43 tiles per item, ~36 stages per paged range
    check([int(x) for x in rng.integers(128, 2049, 256)], [0] * 256, [16384], 5, hkv=2, hq=10)
    # 14B-shaped share, 128 requests: 43 tiles, ~68 stages
    check([int(x) for x in rng.integers(128, 4097, 128)], [0] * 128, [16384], 3, hkv=4, hq=20)
    # eight groups of 16 (tiles of 2 row waves): always 3
    lens = [int(x) for x in rng.integers(128, 4097, 128)]
    check(lens, [g for g in range(8) for _ in range(16)], [12134, 14070, 6942, 11971, 5849, 5146, 4709, 3846], 3)
    assert int(batch_of([300] * 64, [0] * 64, [200]).plan().co_prefix_stages) == 0   # not co-resident


def test_two_launches_by_parameter():
    p = R.default_params()
    assert p.single_launch == 1
