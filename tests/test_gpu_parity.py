"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Allocator outputs (slots, copy-on-write pairs, block tables) and pool
contents are compared bit for bit; attention outputs within the fp32 bound
(max abs 2e-3) plus tighter LSE / relative-error discriminators.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle.attention import decode_reference
from oracle.driver import run_single_step
from shared_prefix_paged_amd import runtime as R
from shared_prefix_paged_amd import _abi as A
from hip_setup import setup_single_step, errors, pool_bytes, to_device

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE, TOL_REL = 2e-3, 1e-3, 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def small_cases():
    return {
        "c0": lambda: W.make_workload(W.CONFIGS["C0"]),
        "bf16_d128_g4_multi": lambda: W.make_custom(
            batch=7, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", group_prefix_len=[40, 17],
            group_of=[0, 0, 1, -1, 1, 0, 1], suffix_len=[5, 1, 33, 9, 16, 17, 2], seed=11),
        "bf16_d64_g2": lambda: W.make_custom(
            batch=5, num_q_heads=6, num_kv_heads=3, head_dim=64, dtype="bf16", group_prefix_len=[129],
            group_of=[0, 0, 0, 0, 0], suffix_len=[1, 64, 65, 200, 3], seed=12),
        "bf16_d128_g5_tail": lambda: W.make_custom(
            batch=9, num_q_heads=10, num_kv_heads=2, head_dim=128, dtype="bf16", group_prefix_len=[300],
            group_of=[0] * 9, suffix_len=[7, 300, 1, 45, 130, 2, 99, 64, 17], seed=13),
        "bf16_d128_g8": lambda: W.make_custom(
            batch=6, num_q_heads=8, num_kv_heads=1, head_dim=128, dtype="bf16", group_prefix_len=[77, 500],
            group_of=[1, 1, 0, 1, 0, -1], suffix_len=[3, 8, 1, 250, 31, 12], seed=14),
        "bf16_d128_mha": lambda: W.make_custom(
            batch=4, num_q_heads=4, num_kv_heads=4, head_dim=128, dtype="bf16", group_prefix_len=[64],
            group_of=[0, 0, 0, 0], suffix_len=[9, 10, 11, 12], seed=15),
        "f32_d128_g3": lambda: W.make_custom(
            batch=5, num_q_heads=6, num_kv_heads=2, head_dim=128, dtype="f32", group_prefix_len=[90],
            group_of=[0, 0, -1, 0, 0], suffix_len=[4, 70, 5, 1, 33], seed=16),
        "bf16_many_tiles": lambda: W.make_custom(
            batch=40, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", group_prefix_len=[1000],
            group_of=[0] * 40, suffix_len=list(np.random.default_rng(5).integers(1, 3000, 40)), seed=17),
        "bf16_hkv16": lambda: W.make_custom(
            batch=3, num_q_heads=16, num_kv_heads=16, head_dim=64, dtype="bf16", group_prefix_len=[33],
            group_of=[0, 0, 0], suffix_len=[5, 6, 400], seed=18),
        # the remaining query-rows-per-head counts of the bf16 paged pass (3, 6, 7)
        "bf16_d128_g3": lambda: W.make_custom(
            batch=6, num_q_heads=6, num_kv_heads=2, head_dim=128, dtype="bf16", group_prefix_len=[260],
            group_of=[0, -1, 0, 0, -1, 0], suffix_len=[15, 81, 16, 1, 17, 129], seed=19),
        "bf16_d128_g6": lambda: W.make_custom(
            batch=5, num_q_heads=12, num_kv_heads=2, head_dim=128, dtype="bf16", group_prefix_len=[48],
            group_of=[0, 0, -1, 0, 0], suffix_len=[63, 64, 65, 2, 200], seed=20),
        "bf16_d64_g7": lambda: W.make_custom(
            batch=4, num_q_heads=7, num_kv_heads=1, head_dim=64, dtype="bf16", group_prefix_len=[700],
            group_of=[0, 0, 0, -1], suffix_len=[31, 1, 500, 47], seed=21),
        # groups of more than 64 query rows take the two-key-half prefix tiles:
        # a last chunk of one 32-key tile (second half idle), an odd tile count,
        # and a prefix shorter than one tile
        "bf16_d128_halves_ragged": lambda: W.make_custom(
            batch=24, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16", group_prefix_len=[276, 326, 21],
            group_of=[0] * 18 + [1, 1, 2, 2, -1, 1], suffix_len=list(range(1, 25)), seed=22),
        "bf16_d64_halves_ragged": lambda: W.make_custom(
            batch=11, num_q_heads=8, num_kv_heads=1, head_dim=64, dtype="bf16", group_prefix_len=[545, 7],
            group_of=[0] * 9 + [1, 1], suffix_len=[3, 70, 1, 5, 9, 130, 2, 33, 64, 17, 8], seed=23),
        # more requests than one paged-pass launch takes (256): two sub-batches,
        # each with its own stream-K split and merge launch
        "bf16_two_sub_batches": lambda: W.make_custom(
            batch=300, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", group_prefix_len=[96, 31, 700],
            group_of=[int(g) for g in np.random.default_rng(24).integers(-1, 3, 300)],
            suffix_len=[int(x) for x in np.random.default_rng(25).integers(1, 90, 300)], seed=24),
        # float32 prefix contraction: several 32-row tiles per group and
        # head, several key splits, a ragged last tile, two groups
        "f32_many_rows": lambda: W.make_custom(
            batch=45, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="f32", group_prefix_len=[3001, 40],
            group_of=[0] * 40 + [1, 1, 1, -1, 0], suffix_len=[int(x) for x in np.random.default_rng(28).integers(1, 90, 45)],
            seed=26),
        # the most groups a step takes (512): most groups with one or two
        # members, some with none, a few requests without a prefix; more
        # requests than one paged-pass launch takes
        "bf16_512_groups": lambda: W.make_custom(
            batch=700, num_q_heads=4, num_kv_heads=2, head_dim=64, dtype="bf16",
            group_prefix_len=[int(x) for x in np.random.default_rng(29).integers(1, 70, 512)],
            group_of=[-1 if i % 97 == 0 else int(g)
                      for i, g in enumerate(np.random.default_rng(30).integers(0, 512, 700))],
            suffix_len=[int(x) for x in np.random.default_rng(31).integers(1, 20, 700)], seed=27),
        "f32_two_sub_batches": lambda: W.make_custom(
            batch=260, num_q_heads=4, num_kv_heads=1, head_dim=64, dtype="f32", group_prefix_len=[50, 130],
            group_of=[int(g) for g in np.random.default_rng(26).integers(-1, 2, 260)],
            suffix_len=[int(x) for x in np.random.default_rng(27).integers(1, 40, 260)], seed=25),
    }


CASES = small_cases()


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    note(f"[setup] case={request.param}")
    wl = CASES[request.param]()
    ref = decode_reference(wl)
    return request.param, wl, ref


def test_allocator_outputs_bit_exact(case):
    name, wl, _ = case
    st_o = run_single_step(wl, with_mirror=False)
    note(f"[gpu] setup {name}")
    st = setup_single_step(wl)
    torch.cuda.synchronize()
    assert list(st.setup_slots) == st_o.setup_slots
    assert list(st.step_slots) == st_o.step_slots
    assert st.step_cows == st_o.step_cows
    assert st.bases == st_o.bases
    for b in range(wl.batch):
        n = len(st_o.tables[b])
        assert list(st.tables[b, :n]) == st_o.tables[b] and np.all(st.tables[b, n:] == -1)
        assert st.lens[b] == st_o.lens[b]
    assert st.cold.state() == st_o.cold.state()
    assert st.hot.state() == st_o.hot.state()


def test_pools_byte_exact(case):
    name, wl, _ = case
    st_o = run_single_step(wl)
    note(f"[gpu] pools {name}")
    st = setup_single_step(wl)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pool_bytes(st.pools.k_hot)[:st_o.mirror.k_hot.size], st_o.mirror.k_hot)
    np.testing.assert_array_equal(pool_bytes(st.pools.v_hot)[:st_o.mirror.v_hot.size], st_o.mirror.v_hot)
    np.testing.assert_array_equal(pool_bytes(st.pools.k_cold), st_o.mirror.k_cold)
    np.testing.assert_array_equal(pool_bytes(st.pools.v_cold), st_o.mirror.v_cold)


@pytest.mark.parametrize("mode", ["cascade", "dense", "step_per_group", "step_batch_global"])
def test_attention_matches_oracle(case, mode):
    name, wl, (ref_o, ref_l) = case
    note(f"[gpu] attention {name} {mode}")
    st = setup_single_step(wl)
    ws = R.workspace(st.batch)
    if mode == "cascade":
        out, lse = R.cascade_decode(st.batch, st.pools, ws)
    elif mode == "dense":
        out, lse = R.dense_decode(st.batch, st.pools, ws)
    else:
        m = A.SPKV_MODE_PER_GROUP if mode == "step_per_group" else A.SPKV_MODE_BATCH_GLOBAL
        out, lse, _ = R.decode_step(st.batch, st.pools, R.default_params(m), ws)
    torch.cuda.synchronize()
    e_o, e_l, rel = errors(out, lse, ref_o, ref_l)
    note(f"    max_abs={e_o:.3e} lse={e_l:.3e} rel={rel:.3e}")
    assert e_o <= TOL_O and e_l <= TOL_LSE and rel <= TOL_REL


def test_cascade_deterministic(case):
    name, wl, _ = case
    note(f"[gpu] determinism {name}")
    st = setup_single_step(wl)
    ws = R.workspace(st.batch)
    o1, l1 = R.cascade_decode(st.batch, st.pools, ws)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = R.cascade_decode(st.batch, st.pools, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_page_size_16_and_reshuffle_match():
    wl = CASES["bf16_d128_g4_multi"]()
    ref_o, ref_l = decode_reference(wl)
    outs = []
    for P, fo in [(1, None), (16, None), (16, "perm"), (4, "perm")]:
        w = W.make_custom(batch=7, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16",
                          group_prefix_len=[40, 17], group_of=[0, 0, 1, -1, 1, 0, 1],
                          suffix_len=[5, 1, 33, 9, 16, 17, 2], seed=11, page_size=P)
        order = None if fo is None else np.random.default_rng(P).permutation(w.num_cold_pages).astype(np.int32)
        note(f"[gpu] page size {P} order={fo}")
        st = setup_single_step(w, page_size=P, free_order=order)
        ws = R.workspace(st.batch)
        out, lse = R.cascade_decode(st.batch, st.pools, ws)
        torch.cuda.synchronize()
        e_o, e_l, _ = errors(out, lse, ref_o, ref_l)
        assert e_o <= TOL_O and e_l <= TOL_LSE
        outs.append(out.cpu())
    # the same logical tokens in a different physical order give the same reduction order here
    for o in outs[1:]:
        assert torch.allclose(o, outs[0], atol=1e-6, rtol=0)


def test_merge_states_kernel():
    rng = np.random.default_rng(4)
    rows, d = 37, 128
    oa, ob = rng.standard_normal((rows, d)), rng.standard_normal((rows, d))
    la, lb = rng.standard_normal(rows) * 3, rng.standard_normal(rows) * 3
    la[3] = -np.inf
    la[5] = lb[5] = -np.inf
    from oracle.attention import merge
    ro, rl = merge(oa, la, ob, lb)
    t = lambda x: torch.tensor(x, dtype=torch.float32, device="cuda")
    note("[gpu] merge_states")
    o, l = R.merge_states(t(oa), t(la), t(ob), t(lb))
    torch.cuda.synchronize()
    np.testing.assert_allclose(o.cpu().numpy(), ro, atol=1e-5)
    lg = l.cpu().numpy()
    assert np.isneginf(lg[5]) and np.allclose(lg[np.isfinite(rl)], rl[np.isfinite(rl)], atol=1e-5)


def test_empty_batch_and_no_groups():
    wl = W.make_custom(batch=3, num_q_heads=4, num_kv_heads=1, head_dim=64, dtype="bf16", group_prefix_len=[],
                       group_of=[-1, -1, -1], suffix_len=[1, 2, 300], seed=21)
    ref_o, ref_l = decode_reference(wl)
    note("[gpu] no groups")
    st = setup_single_step(wl)
    ws = R.workspace(st.batch)
    out, lse = R.cascade_decode(st.batch, st.pools, ws)
    torch.cuda.synchronize()
    e_o, e_l, _ = errors(out, lse, ref_o, ref_l)
    assert e_o <= TOL_O and e_l <= TOL_LSE


# ---------------------------------------------------------------- full-size configs (every row)

def full_size(name, **kw):
    return W.make_workload(W.CONFIGS[name], **kw)


def v_bounds(wl):
    """Per (request, query head, dim): min and max of the V values the row
    attends (its group's HOT prefix and its own suffix), float64."""
    from oracle.attention import widen
    cfg = wl.cfg
    G, hkv = cfg.group_size, cfg.num_kv_heads
    B, Hq, d = wl.q.shape
    lo = np.empty((B, Hq, d))
    hi = np.empty((B, Hq, d))
    pre = [(widen(v, cfg.dtype).min(axis=0), widen(v, cfg.dtype).max(axis=0)) for v in wl.prefix_v]
    for b in range(B):
        sv = widen(wl.suffix_kv(b)[1], cfg.dtype)
        mn, mx = sv.min(axis=0), sv.max(axis=0)          # [Hkv, d]
        g = int(wl.group_of[b])
        if g >= 0:
            mn, mx = np.minimum(mn, pre[g][0]), np.maximum(mx, pre[g][1])
        lo[b] = np.repeat(mn, G, axis=0)
        hi[b] = np.repeat(mx, G, axis=0)
    return lo, hi


FULL = [("C1", None), ("C2", None)] + [("C3", lp) for lp in W.C3_LP_SWEEP] + [("C3", lp) for lp in W.C3_LP_LOW]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,lp", FULL)
def test_full_size_every_row(name, lp):
    # BASELINE configurations at full size, in the launch configuration the
    # benchmark times: every row against the oracle (grouped form: one prefix
    # product per group), for the cascade, the flat pass and the dispatcher's
    # per-group choice.  Property at any size: each output is a convex
    # combination of the V rows it attends, so it lies within their per-dim
    # min / max (the kernels normalise by the weights they apply; the flat
    # pass's hi + lo weights carry ~16 bits, hence the small slack).
    from oracle.attention import decode_reference_grouped
    note(f"[gpu] full size {name} lp={lp}: drawing")
    wl = full_size(name, prefix_len=lp)
    ref_o, ref_l = decode_reference_grouped(wl)
    lo, hi = v_bounds(wl)
    note(f"[gpu] full size {name} lp={lp}: B={wl.batch} groups={len(wl.group_prefix_len)} setup")
    st = setup_single_step(wl)
    ws = R.workspace(st.batch)
    def fused():
        # the benchmark's launch: the step's token read from k_new / v_new and
        # landed by the merge launch (the same bytes at the same slot as the
        # setup wrote), from the device lengths before the append
        off = wl.suffix_offsets
        k_new = to_device(wl.suffix_k[off[1:] - 1], wl.cfg.dtype)
        v_new = to_device(wl.suffix_v[off[1:] - 1], wl.cfg.dtype)
        st.batch.lens -= 1
        out, lse, _ = R.decode_step_append(st.batch, st.pools, R.default_params(A.SPKV_MODE_PER_GROUP), ws,
                                           k_new, v_new, st.step_slots)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(st.batch.lens.cpu().numpy(), st.lens)     # lengths advanced once
        np.testing.assert_array_equal(st.batch.tables.cpu().numpy().reshape(st.tables.shape), st.tables)
        return out, lse

    runs = [("cascade", lambda: R.cascade_decode(st.batch, st.pools, ws)),
            ("dense", lambda: R.dense_decode(st.batch, st.pools, ws)),
            ("step_per_group", lambda: R.decode_step(st.batch, st.pools, R.default_params(A.SPKV_MODE_PER_GROUP), ws)[:2])]
    if wl.cfg.dtype == "bf16":
        runs.append(("step_append_fused", fused))
    for mode, fn in runs:
        out, lse = fn()
        torch.cuda.synchronize()
        e_o, e_l, rel = errors(out, lse, ref_o, ref_l)
        o = out.cpu().double().numpy()
        slack = 1e-4 * np.maximum(np.abs(lo), np.abs(hi)) + 1e-6
        outside = int(np.sum((o < lo - slack) | (o > hi + slack)))
        note(f"    {mode}: max_abs={e_o:.3e} lse={e_l:.3e} rel={rel:.3e} outside_hull={outside}")
        assert e_o <= TOL_O and e_l <= TOL_LSE and rel <= TOL_REL
        assert outside == 0


@pytest.mark.parametrize("P", [1, 16])
def test_cold_fallback_matches_admitted_prefix(P):
    # [GKV] Appendix B.10: a prefix that finds no room in the HOT pool stays in
    # COLD as each of its requests' own leading tokens (private copies), and
    # those requests take the paged pass.  Their attention must be what the
    # admitted prefix gives: group 1 below is not admitted, group 0 is.
    note(f"[gpu] COLD fallback P={P}")
    wl = W.make_custom(batch=10, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16",
                       group_prefix_len=[300, 45], group_of=[0, 0, 1, 0, 1, 1, 0, -1, 0, 1],
                       suffix_len=[5, 17, 1, 40, 16, 33, 2, 9, 64, 3], page_size=P, seed=61)
    ref_o, ref_l = decode_reference(wl)
    moved = wl.group_of == 1
    ks, vs, ls = [], [], []
    for b in range(wl.batch):
        sk, sv = wl.suffix_kv(b)
        if moved[b]:
            sk, sv = np.concatenate([wl.prefix_k[1], sk]), np.concatenate([wl.prefix_v[1], sv])
        ks.append(sk)
        vs.append(sv)
        ls.append(len(sk))
    ls = np.asarray(ls, np.int64)
    pages = W.cold_pages_for(int(ls.sum()), wl.batch, P)
    fb = dataclasses.replace(
        wl, cfg=dataclasses.replace(wl.cfg, num_groups=1), group_prefix_len=wl.group_prefix_len[:1],
        prefix_k=wl.prefix_k[:1], prefix_v=wl.prefix_v[:1], group_of=np.where(moved, -1, wl.group_of).astype(np.int32),
        suffix_len=ls, suffix_k=np.concatenate(ks), suffix_v=np.concatenate(vs), suffix_offsets=None,
        num_cold_pages=pages, free_order=np.random.default_rng(62).permutation(pages).astype(np.int32),
        hot_capacity=int(wl.group_prefix_len[0]))
    fb.__post_init__()
    st = setup_single_step(fb)
    ws = R.workspace(st.batch)
    for mode, fn in (("cascade", lambda: R.cascade_decode(st.batch, st.pools, ws)),
                     ("dense", lambda: R.dense_decode(st.batch, st.pools, ws)),
                     ("per_group", lambda: R.decode_step(st.batch, st.pools, R.default_params(A.SPKV_MODE_PER_GROUP), ws)[:2])):
        out, lse = fn()
        torch.cuda.synchronize()
        e_o, e_l, rel = errors(out, lse, ref_o, ref_l)
        note(f"    {mode}: max_abs={e_o:.2e} lse={e_l:.2e} rel={rel:.2e}")
        assert e_o <= TOL_O and e_l <= TOL_LSE and rel <= TOL_REL


def _single_launch_cases():
    rng = np.random.default_rng(64)
    return {
        "one_group_8_heads": lambda: CASES["bf16_many_tiles"](),
        "two_groups_4_heads": lambda: W.make_custom(
            batch=70, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16", group_prefix_len=[700, 2000],
            group_of=[0] * 30 + [1] * 36 + [-1] * 4, suffix_len=[int(x) for x in rng.integers(1, 300, 70)],
            seed=63),
        # groups of 33..64 query rows per KV head: prefix tiles of 2 row waves (4 of the 8 waves)
        "two_groups_2_wave_tiles": lambda: W.make_custom(
            batch=33, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", group_prefix_len=[3000, 5000],
            group_of=[0] * 16 + [1] * 16 + [-1], suffix_len=[int(x) for x in rng.integers(1, 600, 33)], seed=67),
        # KV heads beyond one group of 4: the last paged head group partly filled (6), and the most (16)
        "one_group_6_heads": lambda: W.make_custom(
            batch=41, num_q_heads=12, num_kv_heads=6, head_dim=128, dtype="bf16", group_prefix_len=[1200],
            group_of=[0] * 40 + [-1], suffix_len=[int(x) for x in rng.integers(1, 300, 41)], seed=68),
        "one_group_16_heads": lambda: W.make_custom(
            batch=100, num_q_heads=16, num_kv_heads=16, head_dim=128, dtype="bf16", group_prefix_len=[700],
            group_of=[0] * 100, suffix_len=[int(x) for x in rng.integers(1, 200, 100)], seed=69),
        # fewer than 4 KV heads: 2 or 4 paged blocks side by side in one launch block
        "one_group_2_heads": lambda: W.make_custom(
            batch=61, num_q_heads=10, num_kv_heads=2, head_dim=128, dtype="bf16", group_prefix_len=[1500],
            group_of=[0] * 60 + [-1], suffix_len=[int(x) for x in rng.integers(1, 400, 61)], seed=65),
        "one_group_1_head": lambda: W.make_custom(
            batch=41, num_q_heads=4, num_kv_heads=1, head_dim=128, dtype="bf16", group_prefix_len=[900],
            group_of=[0] * 40 + [-1], suffix_len=[int(x) for x in rng.integers(1, 500, 41)], seed=66),
        # the deep, pipelined prefix ring with items of 1, 2 and 3 key tiles (the last chunks of
        # 513-, 576- and 608-key prefixes) beside 8-tile items
        "deep_ring_short_items": lambda: W.make_custom(
            batch=36, num_q_heads=64, num_kv_heads=8, head_dim=128, dtype="bf16", group_prefix_len=[513, 576, 608],
            group_of=[0] * 12 + [1] * 12 + [2] * 12, suffix_len=[int(x) for x in rng.integers(40, 89, 36)],
            seed=71),
        # one large group beside seven single-request groups: every group counted at the large one's
        # 4 row tiles gives more prefix items than paged blocks, so the one launch is not co-resident
        "uneven_groups_not_co_resident": lambda: W.make_custom(
            batch=107, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
            group_prefix_len=[2000, 1800, 2100, 1900, 2200, 1700, 2300, 1600],
            group_of=[0] * 100 + [1, 2, 3, 4, 5, 6, 7], suffix_len=[int(x) for x in rng.integers(1, 100, 107)],
            seed=70),
    }

# co_resident of each case's plan (every group on the cascade)
SINGLE_CO = {name: name != "uneven_groups_not_co_resident" for name in _single_launch_cases()}


SINGLE = _single_launch_cases()


@pytest.mark.parametrize("name", sorted(SINGLE))
def test_single_launch_matches_two_launches(name):
    # paged_prefix_kernel (single_launch = 2) runs the paged pass's ranges and
    # the prefix blocks of the same plan in one launch: outputs bit-identical
    # to the two launches (single_launch = 0), for the decode step and for the
    # step with fused appends (pools, block tables and lengths too), and both
    # within the bound of the oracle.  The default (single_launch = 1) runs
    # paged_prefix_co_kernel, both roles side by side in every launch block,
    # where the plan marks it co-resident, else paged_prefix_kernel.
    note(f"[gpu] single launch {name}")
    wl = SINGLE[name]()
    ref_o, ref_l = decode_reference(wl)
    states = [setup_single_step(wl, max_blocks=int(wl.suffix_len.max()) + 4) for _ in range(3)]
    info = states[0].batch.plan()
    assert int(info.single_launch) == 1 and int(info.co_resident) == int(SINGLE_CO[name])
    if name == "deep_ring_short_items":
        assert int(info.co_prefix_stages) == 5   # the pipelined prefix loop
    res = []
    for one, st in zip((2, 0, 1), states):
        params = R.default_params(A.SPKV_MODE_FORCE_CASCADE)
        params.single_launch = one
        ws = R.workspace(st.batch)
        with R.KernelTimer() as kt:
            out, lse, _ = R.decode_step(st.batch, st.pools, params, ws)
            torch.cuda.synchronize()
            n_single, n_paged = kt.read(A.SPKV_KERNEL_PAGED_PREFIX)[1], kt.read(A.SPKV_KERNEL_FLAT)[1]
        assert (n_single, n_paged) == ((1, 0) if one else (0, 1))
        e_o, e_l, rel = errors(out, lse, ref_o, ref_l)
        note(f"    single_launch={one}: max_abs={e_o:.2e} lse={e_l:.2e} rel={rel:.2e}")
        assert e_o <= TOL_O and e_l <= TOL_LSE and rel <= TOL_REL
        # one more step with the appends fused in, from identical states
        dr = W.step_draws(wl.cfg, 1, wl.batch)
        k, v, q = (to_device(x, wl.cfg.dtype, "cuda") for x in (dr.k_new, dr.v_new, dr.q))
        slots, cows = st.cold.append_batch(np.asarray(st.seqs, np.int32))
        assert not cows
        st.batch.lens_h += 1
        st.batch.struct.q = q.data_ptr()
        out2, lse2, _ = R.decode_step_append(st.batch, st.pools, params, R.workspace(st.batch), k, v, slots)
        torch.cuda.synchronize()
        res.append((out, lse, out2, lse2))
    for x, y in zip(res[0], res[1]):
        assert torch.equal(x, y)
    # the co-resident launch runs each prefix item in one key half instead of
    # two (another online-softmax reference, so other bf16 roundings of the
    # weights): within the oracle's bound of the two launches; without it the
    # default is paged_prefix_kernel, bit-identical
    for x, y in zip(res[2], res[1]):
        if not SINGLE_CO[name]:
            assert torch.equal(x, y)
            continue
        fin = torch.isfinite(y)
        assert torch.equal(fin, torch.isfinite(x))
        assert float((x[fin] - y[fin]).abs().max()) <= TOL_O
    a, b, c = states
    for t0, t1, t2 in ((a.pools.k_cold, b.pools.k_cold, c.pools.k_cold),
                       (a.pools.v_cold, b.pools.v_cold, c.pools.v_cold)):
        np.testing.assert_array_equal(pool_bytes(t0), pool_bytes(t1))
        np.testing.assert_array_equal(pool_bytes(t2), pool_bytes(t1))
    for st in (a, c):
        assert torch.equal(st.batch.tables, b.batch.tables) and torch.equal(st.batch.lens, b.batch.lens)


@pytest.mark.parametrize("d", [128, 64])
def test_prefix_only_requests_and_a_64k_prefix(d):
    # Degenerate lengths: requests whose whole context is their group's
    # prefix (no COLD token: the suffix part is empty, weight 0 in Eq. (1)),
    # a request with neither (zero output, log-sum-exp -inf), and one group
    # with a 65536-token prefix (key chunks at the 64-split cap), in every mode.
    # Rows of that group merge more partial states than one load batch holds
    # (over 40), so the merge's later batches rescale what the first summed.
    note(f"[gpu] prefix-only requests, 64K prefix, d={d}")
    suffix = [0, 7, 0, 300, 1, 0, 45, 0]
    wl = W.make_custom(batch=8, num_q_heads=8, num_kv_heads=2, head_dim=d, dtype="bf16",
                       group_prefix_len=[65536, 700], group_of=[0, 0, 1, 1, 0, -1, 1, 0], suffix_len=suffix, seed=70)
    ref_o, ref_l = decode_reference(wl)
    st = setup_single_step(wl)            # appends at least one token per request ...
    zero = np.asarray(suffix) == 0
    st.batch.lens_h[zero] = 0             # ... so the empty suffixes are set afterwards, host and device
    st.batch.lens.copy_(torch.from_numpy(st.batch.lens_h).to(st.batch.lens.device))
    ws = R.workspace(st.batch)
    fp, pp = st.batch.plan_parts([1, 1])
    assert int((fp + pp).max()) > 40, "a row merges more partials than one load batch"
    for mode, fn in (("cascade", lambda: R.cascade_decode(st.batch, st.pools, ws)),
                     ("dense", lambda: R.dense_decode(st.batch, st.pools, ws)),
                     ("per_group", lambda: R.decode_step(st.batch, st.pools, R.default_params(A.SPKV_MODE_PER_GROUP), ws)[:2])):
        out, lse = fn()
        torch.cuda.synchronize()
        o, l = out.cpu().double().numpy(), lse.cpu().double().numpy()
        assert np.all(o[5] == 0) and np.all(np.isneginf(l[5])), f"{mode}: empty context"
        keep = np.arange(8) != 5
        e_o = np.abs(o[keep] - ref_o[keep]).max()
        e_l = np.abs(l[keep] - ref_l[keep]).max()
        note(f"    {mode}: max_abs={e_o:.2e} lse={e_l:.2e}")
        assert e_o <= TOL_O and e_l <= TOL_LSE
