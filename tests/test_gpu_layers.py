"""Several layers in one HOT and one COLD allocation (needs an MI355X).

GraniKV paper, Section 3.2: a prefix's HOT slab holds every layer, head h of
layer l at row base*Hkv*L + l*Lp*Hkv + h*Lp; the COLD pool is layer-major with
the same slots and block tables in every layer ("Paged KV cache" page, How it
works).  L = 4 layers drawn independently with the same lengths go through one
allocator: pool bytes of every layer equal the oracle mirror's, attention at
every layer equals the oracle on that layer's tokens, and a fork followed by
appends at page size 16 copies the shared page in every layer.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle.alloc import ColdPool as OColdPool, HotPool as OHotPool
from oracle.attention import decode_reference_grouped
from oracle.pools import PoolMirror
from shared_prefix_paged_amd import runtime as R
from shared_prefix_paged_amd import _abi as A
from hip_setup import to_device, errors, pool_bytes

pytestmark = pytest.mark.gpu

L = 4
TOL_O, TOL_LSE, TOL_REL = 2e-3, 1e-3, 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def layer_workloads(P):
    kw = dict(batch=12, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", group_prefix_len=[300, 70],
              group_of=[0, 0, 1, 0, -1, 1, 0, 0, 1, 0, 0, 1],
              suffix_len=[17, 40, 3, 200, 33, 16, 1, 95, 64, 18, 130, 7], page_size=P, extra_steps=8)
    return [W.make_custom(seed=60 + l, **kw) for l in range(L)]


def test_four_layers_share_one_allocation():
    P = 16
    wls = layer_workloads(P)
    wl0 = wls[0]
    cfg = wl0.cfg
    B, hkv, d = wl0.batch, cfg.num_kv_heads, cfg.head_dim
    fo = list(wl0.free_order)

    # host allocators (native) and the oracle's, driven identically
    hot, ohot = R.HotPool(wl0.hot_capacity), OHotPool(wl0.hot_capacity)
    members = np.bincount(wl0.group_of[wl0.group_of >= 0], minlength=2)
    bases = []
    for g, lp in enumerate(wl0.group_prefix_len):
        b, ob = hot.alloc(int(lp)), ohot.alloc(int(lp))
        assert b == ob
        for _ in range(int(members[g]) - 1):
            hot.incref(b)
            ohot.incref(ob)
        bases.append(b)
    cold, ocold = R.ColdPool(wl0.num_cold_pages, P, fo), OColdPool(wl0.num_cold_pages, P, fo)
    seqs = [cold.seq_new() for _ in range(B)]
    for _ in range(B):
        ocold.seq_new()
    ids = [b for b in range(B) for _ in range(int(wl0.suffix_len[b]))]
    slots, cows = cold.append_batch(ids)
    oslots, ocows, _, err = ocold.append_batch(ids)
    assert err is None and list(slots) == oslots and cows == [] == ocows

    note("[gpu] layers: writing 4 layers")
    pools = R.KVPools.allocate(wl0.hot_capacity, wl0.num_cold_pages * P, hkv, d, torch.bfloat16, num_layers=L)
    mirror = PoolMirror(wl0.hot_capacity, wl0.num_cold_pages * P, hkv, d, np.uint16, num_layers=L)
    for l, wl in enumerate(wls):
        for g, base in enumerate(bases):
            R.hot_write(to_device(wl.prefix_k[g], "bf16"), to_device(wl.prefix_v[g], "bf16"), base, pools.k_hot,
                        pools.v_hot, wl0.hot_capacity, hkv, d, num_layers=L, layer=l)
            mirror.hot_write(wl.prefix_k[g], wl.prefix_v[g], base, layer=l)
        kc, vc = pools.cold_layer(l)
        R.reshape_and_cache(to_device(wl.suffix_k, "bf16"), to_device(wl.suffix_v, "bf16"),
                            torch.from_numpy(np.asarray(slots, np.int32)).cuda(), kc, vc, pools.cold_slots, hkv, d)
        mirror.reshape_and_cache(wl.suffix_k, wl.suffix_v, slots, layer=l)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pool_bytes(pools.k_hot), mirror.k_hot)
    np.testing.assert_array_equal(pool_bytes(pools.v_hot), mirror.v_hot)
    np.testing.assert_array_equal(pool_bytes(pools.k_cold), mirror.k_cold)
    np.testing.assert_array_equal(pool_bytes(pools.v_cold), mirror.v_cold)

    tables, lens = cold.block_tables(seqs, max(1, -(-int(wl0.suffix_len.max()) // P)) + 2)
    for l, wl in enumerate(wls):
        ref_o, ref_l = decode_reference_grouped(wl)
        batch = R.DecodeBatch(to_device(wl.q, "bf16"), wl.group_of, bases, wl.group_prefix_len, tables, lens, P, hkv)
        ws = R.workspace(batch)
        kv = pools.at_layer(l)
        for mode, fn in (("cascade", lambda: R.cascade_decode(batch, kv, ws)),
                         ("dense", lambda: R.dense_decode(batch, kv, ws)),
                         ("step", lambda: R.decode_step(batch, kv, R.default_params(A.SPKV_MODE_PER_GROUP), ws)[:2])):
            out, lse = fn()
            torch.cuda.synchronize()
            e_o, e_l, rel = errors(out, lse, ref_o, ref_l)
            note(f"    layer {l} {mode}: max_abs={e_o:.2e} lse={e_l:.2e} rel={rel:.2e}")
            assert e_o <= TOL_O and e_l <= TOL_LSE and rel <= TOL_REL

    # Fork request 3 (a partially filled last page at P = 16), append one token
    # to parent and child: the parent's append copies the shared page, in every
    # layer, before the new tokens land.
    parent = 3
    child, ochild = cold.fork(parent), ocold.fork(parent)
    assert child == ochild
    s2, c2 = cold.append_batch([parent, child])
    os2, oc2, _, err = ocold.append_batch([parent, child])
    assert err is None and list(s2) == os2 and c2 == oc2 and len(c2) == 1
    R.copy_blocks(torch.tensor(c2, dtype=torch.int32, device="cuda"), pools.k_cold, pools.v_cold,
                  wl0.num_cold_pages, P, hkv, d, num_layers=L)
    mirror.copy_blocks(c2, P)
    new = [W.step_draws(wl.cfg, 1, 2) for wl in wls]
    for l in range(L):
        kc, vc = pools.cold_layer(l)
        R.reshape_and_cache(to_device(new[l].k_new, "bf16"), to_device(new[l].v_new, "bf16"),
                            torch.from_numpy(np.asarray(s2, np.int32)).cuda(), kc, vc, pools.cold_slots, hkv, d)
        mirror.reshape_and_cache(new[l].k_new, new[l].v_new, s2, layer=l)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pool_bytes(pools.k_cold), mirror.k_cold)
    np.testing.assert_array_equal(pool_bytes(pools.v_cold), mirror.v_cold)
    # the child's attention at every layer: the parent's history plus its own token
    t2, l2 = cold.block_tables([parent, child], tables.shape[1])
    for l, wl in enumerate(wls):
        sk, sv = wl.suffix_kv(parent)
        ls = np.array([len(sk) + 1, len(sk) + 1], np.int64)
        two = dataclasses.replace(
            wl, group_of=wl.group_of[[parent, parent]], suffix_len=ls, q=new[l].q,
            suffix_k=np.concatenate([sk, new[l].k_new[:1], sk, new[l].k_new[1:]]),
            suffix_v=np.concatenate([sv, new[l].v_new[:1], sv, new[l].v_new[1:]]),
            suffix_offsets=None, cfg=dataclasses.replace(wl.cfg, batch=2))
        two.__post_init__()
        ref_o, ref_l = decode_reference_grouped(two)
        batch = R.DecodeBatch(to_device(new[l].q, "bf16"), two.group_of, bases, wl.group_prefix_len, t2, l2, P, hkv)
        out, lse, _ = R.decode_step(batch, pools.at_layer(l), R.default_params(A.SPKV_MODE_FORCE_CASCADE),
                                    R.workspace(batch))
        torch.cuda.synchronize()
        e_o, e_l, rel = errors(out, lse, ref_o, ref_l)
        note(f"    layer {l} after fork: max_abs={e_o:.2e} lse={e_l:.2e}")
        assert e_o <= TOL_O and e_l <= TOL_LSE and rel <= TOL_REL
