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


def test_append_tokens_rejects_out_of_range_slots():
    # A slot outside the pool is an error reported before any launch: the
    # pool is untouched (and a good call afterwards writes normally).
    from shared_prefix_paged_amd import InvalidArgument
    dev = "cuda"
    hkv, d, P = 1, 64, 1
    k = torch.zeros(8 * hkv * d, dtype=torch.float32, device=dev)
    v = torch.zeros_like(k)
    knew = torch.ones((3, hkv, d), dtype=torch.float32, device=dev)
    for bad in ([-1, 3, 2], [0, 8, 2]):
        with pytest.raises(InvalidArgument):
            R.append_tokens(knew, knew, np.array(bad, np.int32), k, v, 8, P, hkv, d)
    torch.cuda.synchronize()
    assert k.abs().sum().item() == 0 and v.abs().sum().item() == 0
    R.append_tokens(knew, knew, np.array([5, 3, 2], np.int32), k, v, 8, P, hkv, d)
    torch.cuda.synchronize()
    kk = k.view(8, d).cpu().numpy()
    assert kk[[2, 3, 5]].sum() == 3 * d and kk.sum() == 3 * d


# ---------------------------------------------------------------------------
# spkv_decode_step_append: the step's appends fused into the decode step must
# leave the same outputs, pools, block tables and lengths as the separate
# spkv_append_tokens + spkv_decode_step (same bytes read in the same order, so
# bit for bit), over several steps from identical states.

def _fused_cases():
    rng = np.random.default_rng(31)
    return {
        "bf16_d128_groups": lambda: W.make_custom(
            batch=7, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", group_prefix_len=[40, 300],
            group_of=[0, 0, 1, -1, 1, 0, 1], suffix_len=[5, 1, 33, 9, 16, 17, 2], seed=41),
        "bf16_d64_page16": lambda: W.make_custom(
            batch=6, num_q_heads=8, num_kv_heads=1, head_dim=64, dtype="bf16", group_prefix_len=[500],
            group_of=[0, 0, 0, -1, 0, 0], suffix_len=[15, 16, 17, 31, 32, 1], seed=42, page_size=16),
        "bf16_two_sub_batches": lambda: W.make_custom(
            batch=300, num_q_heads=8, num_kv_heads=4, head_dim=64, dtype="bf16", group_prefix_len=[100, 2000],
            group_of=[0] * 150 + [1] * 140 + [-1] * 10,
            suffix_len=[int(x) for x in rng.integers(1, 60, 300)], seed=43),
    }


FUSED = _fused_cases()


@pytest.mark.parametrize("mode", ["per_group", "cascade", "dense"])
@pytest.mark.parametrize("name", sorted(FUSED))
def test_decode_step_append_matches_separate_calls(name, mode):
    from hip_setup import setup_single_step
    from shared_prefix_paged_amd import _abi as A
    note(f"[gpu] decode_step_append {name} {mode}")
    wl = FUSED[name]()
    cfg = wl.cfg
    B, P, hkv, d = wl.batch, cfg.page_size, cfg.num_kv_heads, cfg.head_dim
    steps = 3
    mb = (int(wl.suffix_len.max()) + steps + P - 1) // P + 1
    states = [setup_single_step(wl, max_blocks=mb) for _ in range(2)]
    params = R.default_params({"per_group": A.SPKV_MODE_PER_GROUP, "cascade": A.SPKV_MODE_FORCE_CASCADE,
                               "dense": A.SPKV_MODE_FORCE_DENSE}[mode])
    for step in range(steps):
        dr = W.step_draws(cfg, step + 1, B)
        k, v, q = (to_device(x, cfg.dtype, "cuda") for x in (dr.k_new, dr.v_new, dr.q))
        res = []
        for j, st in enumerate(states):
            slots, cows = st.cold.append_batch(np.asarray(st.seqs, np.int32))
            if cows:
                R.copy_blocks(torch.tensor(cows, dtype=torch.int32, device="cuda"), st.pools.k_cold,
                              st.pools.v_cold, st.cold.num_pages, P, hkv, d)
            if j == 0:          # separate calls: the appends reach the device state first
                R.append_tokens(k, v, slots, st.pools.k_cold, st.pools.v_cold, st.pools.cold_slots, P, hkv, d,
                                tables=st.batch.tables, max_blocks=st.batch.max_blocks, lens=st.batch.lens)
            st.batch.lens_h += 1
            st.batch.struct.q = q.data_ptr()
            ws = R.workspace(st.batch)
            if j == 0:
                out, lse, choice = R.decode_step(st.batch, st.pools, params, ws)
            else:
                out, lse, choice = R.decode_step_append(st.batch, st.pools, params, ws, k, v, slots)
            res.append((out, lse, np.asarray(choice).copy(), np.asarray(slots).copy()))
        torch.cuda.synchronize()
        (o0, l0, c0, s0), (o1, l1, c1, s1) = res
        np.testing.assert_array_equal(s0, s1)
        np.testing.assert_array_equal(c0, c1)
        assert torch.equal(o0, o1) and torch.equal(l0, l1), f"step {step}"
        a, b = states
        for t0, t1 in ((a.pools.k_cold, b.pools.k_cold), (a.pools.v_cold, b.pools.v_cold)):
            np.testing.assert_array_equal(pool_bytes(t0), pool_bytes(t1))
        assert torch.equal(a.batch.tables, b.batch.tables) and torch.equal(a.batch.lens, b.batch.lens)
        # and the device state follows the host allocator
        t_h, l_h = b.cold.block_tables(b.seqs, b.batch.max_blocks)
        np.testing.assert_array_equal(b.batch.tables.cpu().numpy().reshape(B, -1), t_h)
        np.testing.assert_array_equal(b.batch.lens.cpu().numpy(), l_h)


def test_decode_step_append_rejects_bad_slots():
    from hip_setup import setup_single_step
    from shared_prefix_paged_amd import InvalidArgument
    wl = FUSED["bf16_d128_groups"]()
    st = setup_single_step(wl, max_blocks=int(wl.suffix_len.max()) + 4)
    k = torch.zeros((wl.batch, wl.cfg.num_kv_heads, wl.cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    st.batch.lens_h += 1
    ws = R.workspace(st.batch)
    lens_before = st.batch.lens.clone()
    bad = np.zeros(wl.batch, np.int32)
    bad[3] = st.pools.cold_slots                       # one past the pool
    with pytest.raises(InvalidArgument):
        R.decode_step_append(st.batch, st.pools, R.default_params(), ws, k, k, bad)
    torch.cuda.synchronize()
    assert torch.equal(st.batch.lens, lens_before)     # nothing launched
