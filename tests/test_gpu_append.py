"""spkv_append_tokens (one launch: K/V rows to their COLD slots plus the device
block-table update) against the separate reshape_and_cache and
block_table_append operations, byte for byte ("Paged KV cache" page, How it
works steps 1-3; needs an MI355X)."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from shared_prefix_paged_amd import runtime as R
from hip_setup import to_device, pool_bytes

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("P,n,forks", [(1, 64, 0), (16, 300, 5), (4, 513, 2)])
def test_append_tokens_matches_separate_ops(P, n, forks):
    note(f"[gpu] append_tokens P={P} n={n} forks={forks}")
    rng = np.random.default_rng(P * 1000 + n)
    hkv, d = 2, 128
    pages = (n + forks) * (-(-12 // P) + 1) + 64   # every sequence, its copy-on-write pages, slack
    perm = rng.permutation(pages).astype(np.int32)
    pools = [R.ColdPool(pages, P, perm) for _ in range(2)]
    seqs = [[p.seq_new() for _ in range(n)] for p in pools]
    hist = [int(x) for x in rng.integers(1, 9, size=n)]
    for p, ss in zip(pools, seqs):
        ids = [ss[i] for i in range(n) for _ in range(hist[i])]
        p.append_batch(ids)
        for i in range(forks):
            ss.append(p.fork(ss[i]))
    live = seqs[0]
    mb = 16
    dev = "cuda"
    dt = torch.bfloat16
    k_pool = [torch.zeros(pages * P * hkv * d, dtype=dt, device=dev) for _ in range(2)]
    v_pool = [torch.zeros(pages * P * hkv * d, dtype=dt, device=dev) for _ in range(2)]
    tabs, lens = [], []
    for p, ss in zip(pools, seqs):
        t, l = p.block_tables(ss, mb)
        tabs.append(torch.from_numpy(t).to(dev))
        lens.append(torch.from_numpy(l).to(dev))
    order = rng.permutation(len(live)).astype(np.int32)           # rows in shuffled order
    for step in range(3):
        knew = to_device(W.bf16_bits_from_f32(rng.standard_normal((len(live), hkv, d)).astype(np.float32)), "bf16", dev)
        vnew = to_device(W.bf16_bits_from_f32(rng.standard_normal((len(live), hkv, d)).astype(np.float32)), "bf16", dev)
        res = []
        for j, (p, ss) in enumerate(zip(pools, seqs)):
            slots, cows = p.append_batch([ss[r] for r in order])
            if cows:
                R.copy_blocks(torch.tensor(cows, dtype=torch.int32, device=dev), k_pool[j], v_pool[j], pages, P, hkv, d)
            res.append(slots)
            if j == 0:      # separate operations
                sd = torch.from_numpy(np.asarray(slots, np.int32)).to(dev)
                R.reshape_and_cache(knew, vnew, sd, k_pool[j], v_pool[j], pages * P, hkv, d)
                R.block_table_append(tabs[j], mb, lens[j], torch.from_numpy(order).to(dev), sd, P)
            else:           # fused, host slots and rows in the launch
                R.append_tokens(knew, vnew, slots, k_pool[j], v_pool[j], pages * P, P, hkv, d,
                                tables=tabs[j], max_blocks=mb, lens=lens[j], rows=order)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(res[0], res[1])
        np.testing.assert_array_equal(pool_bytes(k_pool[0]), pool_bytes(k_pool[1]))
        np.testing.assert_array_equal(pool_bytes(v_pool[0]), pool_bytes(v_pool[1]))
        np.testing.assert_array_equal(tabs[0].cpu().numpy(), tabs[1].cpu().numpy())
        np.testing.assert_array_equal(lens[0].cpu().numpy(), lens[1].cpu().numpy())
        # and the device tables equal the host allocator's
        t_h, l_h = pools[1].block_tables(live, mb)
        np.testing.assert_array_equal(tabs[1].cpu().numpy(), t_h)
        np.testing.assert_array_equal(lens[1].cpu().numpy(), l_h)


def test_append_tokens_skips_out_of_range_slots():
    dev = "cuda"
    hkv, d, P = 1, 64, 1
    k = torch.zeros(8 * hkv * d, dtype=torch.float32, device=dev)
    v = torch.zeros_like(k)
    knew = torch.ones((3, hkv, d), dtype=torch.float32, device=dev)
    R.append_tokens(knew, knew, np.array([-1, 8, 2], np.int32), k, v, 8, P, hkv, d)
    torch.cuda.synchronize()
    kk = k.view(8, d).cpu().numpy()
    assert kk[2].sum() == d and kk.sum() == d
