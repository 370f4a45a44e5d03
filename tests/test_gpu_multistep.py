"""Multi-step decode on the HIP path against the oracle's multi-step run
(GraniKV paper, Section 4.5 Table 4 and Appendix B.8b setting: several prefix
groups, a fork of every group's first request at step 8, release of the fork
parents at step 24, full teardown).  Every step: slots, copy-on-write pairs,
block tables and lengths are compared bit for bit with the oracle
allocators; attention (per-group dispatch and batch-global dispatch) is
compared with the oracle's flat fp64 attention over each request's logical
history; at the end both pools are empty and every reference is zero
("Paged KV cache" page, Code: fork / release; needs an MI355X)."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle.driver import MultiStepSim
from shared_prefix_paged_amd import runtime as R
from shared_prefix_paged_amd import _abi as A
from hip_setup import to_device, torch_dtype, errors

pytestmark = pytest.mark.gpu

TOL_O, TOL_L, TOL_REL = 2e-3, 1e-3, 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class GpuMultiStep:
    """HIP side of the multi-step run: native allocators, device pools, the
    same operation order as the oracle's MultiStepSim."""

    def __init__(self, wl, P, fork_step=8, release_step=24, device="cuda"):
        cfg = wl.cfg
        self.wl, self.P, self.dev = wl, P, device
        self.fork_step, self.release_step = fork_step, release_step
        hkv, d = cfg.num_kv_heads, cfg.head_dim
        self.hot = R.HotPool(wl.hot_capacity)
        counts = np.bincount(wl.group_of[wl.group_of >= 0], minlength=len(wl.group_prefix_len))
        self.bases = []
        for g, lp in enumerate(wl.group_prefix_len):
            base = self.hot.alloc(int(lp))
            for _ in range(int(counts[g]) - 1):
                self.hot.incref(base)
            self.bases.append(base)
        self.cold = R.ColdPool(wl.num_cold_pages, P, wl.free_order)
        self.pools = R.KVPools.allocate(wl.hot_capacity, wl.num_cold_pages * P, hkv, d, torch_dtype(cfg.dtype), device)
        for g, base in enumerate(self.bases):
            R.hot_write(to_device(wl.prefix_k[g], cfg.dtype, device), to_device(wl.prefix_v[g], cfg.dtype, device),
                        base, self.pools.k_hot, self.pools.v_hot, wl.hot_capacity, hkv, d)
        B = wl.batch
        self.group_of = {}
        self.live = []
        for b in range(B):
            sid = self.cold.seq_new()
            assert sid == b
            self.group_of[sid] = int(wl.group_of[b])
            self.live.append(sid)
        setup_ids = [b for b in range(B) for _ in range(int(wl.suffix_len[b]) - 1)]
        slots, cows = self.cold.append_batch(setup_ids)
        assert not cows
        off = wl.suffix_offsets
        rows = np.concatenate([np.arange(off[b], off[b + 1] - 1) for b in range(B)])
        self.write(wl.suffix_k[rows], wl.suffix_v[rows], slots)
        self.fork_parents = []
        self.step_index = 0

    def write(self, k, v, slots):
        cfg = self.wl.cfg
        if len(slots) == 0:
            return
        R.reshape_and_cache(to_device(k, cfg.dtype, self.dev), to_device(v, cfg.dtype, self.dev),
                            torch.from_numpy(np.asarray(slots, np.int32)).to(self.dev), self.pools.k_cold,
                            self.pools.v_cold, self.pools.cold_slots, cfg.num_kv_heads, cfg.head_dim)

    def step(self, k_new, v_new, write=True):
        s = self.step_index
        cfg = self.wl.cfg
        if s == self.fork_step:
            firsts = {}
            for b in sorted(self.live):
                g = self.group_of[b]
                if g >= 0 and g not in firsts:
                    firsts[g] = b
            for g in sorted(firsts):
                child = self.cold.fork(firsts[g])
                self.hot.incref(self.bases[g])
                self.group_of[child] = g
                self.live.append(child)
                self.fork_parents.append(firsts[g])
        if s == self.release_step:
            for parent in sorted(self.fork_parents):
                self.cold.release(parent)
                g = self.group_of[parent]
                if g >= 0:
                    self.hot.decref(self.bases[g])
                self.live.remove(parent)
        live = sorted(self.live)
        slots, cows = self.cold.append_batch(live)
        if cows:
            R.copy_blocks(torch.tensor(cows, dtype=torch.int32, device=self.dev), self.pools.k_cold,
                          self.pools.v_cold, self.wl.num_cold_pages, self.P, cfg.num_kv_heads, cfg.head_dim)
        if write:
            self.write(k_new, v_new, slots)
        self.step_index += 1
        return live, np.asarray(slots), [tuple(c) for c in cows]

    def batch(self, live, q):
        lens = [self.cold.seq_info(b)[0] for b in live]
        mb = max([(l + self.P - 1) // self.P for l in lens] + [1])
        tables, lens = self.cold.block_tables(live, mb)
        gof = [self.group_of[b] for b in live]
        return R.DecodeBatch(to_device(q, self.wl.cfg.dtype, self.dev), gof, self.bases, self.wl.group_prefix_len,
                             tables, lens, self.P, self.wl.cfg.num_kv_heads), tables, lens


class SharedRows:
    """Copy-on-write invariant on the device ("Paged KV cache" page, Code:
    fork shares pages, a write to a shared page goes to a private copy):
    device copies of the fork parents' pre-fork K/V rows (gathered at their
    slots) and of the HOT pools, taken just before the forks and compared
    after every later step."""

    def __init__(self, gpu, parents):
        self.gpu = gpu
        P = gpu.P
        slots = []
        for b in parents:
            n, _, nb = gpu.cold.seq_info(b)
            t, _ = gpu.cold.block_tables([b], nb)
            slots += [int(t[0][i // P]) * P + i % P for i in range(n)]
        self.idx = torch.tensor(slots, dtype=torch.int64, device=gpu.dev)
        self.ref = self.snapshot()

    def snapshot(self):
        pools = self.gpu.pools
        row = self.gpu.wl.cfg.num_kv_heads * self.gpu.wl.cfg.head_dim
        k = pools.k_cold.view(-1, row).index_select(0, self.idx)
        v = pools.v_cold.view(-1, row).index_select(0, self.idx)
        return k, v, pools.k_hot.clone(), pools.v_hot.clone()

    def unchanged(self):
        return all(torch.equal(a, b) for a, b in zip(self.snapshot(), self.ref))


def run(wl, P, check_rows, modes=(A.SPKV_MODE_PER_GROUP, A.SPKV_MODE_BATCH_GLOBAL), steps=32, seed=5,
        fused=False):
    """fused: the step's tokens are not written beforehand; every attention
    call is spkv_decode_step_append from the pre-append device lengths (the
    block-table entry it writes is already the allocator's, so rewriting it,
    and landing the same token again for the next mode, changes nothing).
    check_rows(step, n_live, rng) -> the rows compared with the oracle (None: all)."""
    sim = MultiStepSim(wl, page_size=P)
    gpu = GpuMultiStep(wl, P)
    rng = np.random.default_rng(seed)
    choices_seen = {m: set() for m in modes}
    shared = None
    for s in range(steps):
        n_live = len(sim.live) + (len(set(g for g in sim.group_of.values() if g >= 0)) if s == sim.fork_step else 0)
        if s == sim.release_step:
            n_live -= len(sim.fork_parents)
        if s == sim.fork_step:
            firsts = {}
            for b in sorted(sim.live):
                if sim.group_of[b] >= 0:
                    firsts.setdefault(sim.group_of[b], b)
            torch.cuda.synchronize()
            shared = SharedRows(gpu, sorted(firsts.values()))
        dr = W.step_draws(wl.cfg, s, n_live)
        rec = sim.step(dr.k_new, dr.v_new)
        live, slots, cows = gpu.step(dr.k_new, dr.v_new, write=not fused)
        assert live == rec.live, f"step {s}: live sets differ"
        np.testing.assert_array_equal(slots, np.asarray(rec.slots), err_msg=f"step {s} slots")
        assert cows == [tuple(c) for c in rec.cows], f"step {s} copy-on-write pairs"
        batch, tables, lens = gpu.batch(live, dr.q)
        for i, b in enumerate(live):
            t = rec.tables[b]
            assert list(tables[i, :len(t)]) == list(t) and int(lens[i]) == rec.lens[b], f"step {s} request {b}"
        rows = check_rows(s, len(live), rng)
        if rows is None:
            ref_o, ref_l = sim.reference_grouped(live, dr.q)
        else:
            ref_o, ref_l = sim.reference(live, dr.q, rows=rows)
        ws = R.workspace(batch)
        for mode in modes:
            out = torch.empty((len(live), wl.cfg.num_q_heads, wl.cfg.head_dim), dtype=torch.float32, device=gpu.dev)
            lse = torch.empty((len(live), wl.cfg.num_q_heads), dtype=torch.float32, device=gpu.dev)
            if fused:
                batch.lens -= 1                                  # the device view before the append
                k_new, v_new = (to_device(x, wl.cfg.dtype, gpu.dev) for x in (dr.k_new, dr.v_new))
                _, _, choice = R.decode_step_append(batch, gpu.pools, R.default_params(mode), ws, k_new, v_new,
                                                    slots, out, lse)
            else:
                _, _, choice = R.decode_step(batch, gpu.pools, R.default_params(mode), ws, out, lse)
            torch.cuda.synchronize()
            if fused:
                np.testing.assert_array_equal(batch.lens.cpu().numpy(), lens, err_msg=f"step {s} device lengths")
            choices_seen[mode].add(tuple(int(c) for c in choice))
            e_o, e_l, rel = errors(out, lse, ref_o, ref_l, rows=rows)
            assert e_o <= TOL_O and e_l <= TOL_L and rel <= TOL_REL, \
                f"step {s} mode {mode}: max_abs {e_o:.2e} lse {e_l:.2e} rel {rel:.2e}"
        if shared is not None:
            torch.cuda.synchronize()
            assert shared.unchanged(), f"step {s}: a pre-fork row or the HOT slab changed"
        if s % 8 == 0 or rows is None:
            note(f"[gpu] multistep P={P} step {s}: {len(live)} live, {len(cows)} CoW pairs, "
                 f"{'all' if rows is None else len(rows)} rows ok")
    evicted_o = sim.finish()
    for b in sorted(gpu.live):
        gpu.cold.release(b)
        g = gpu.group_of[b]
        if g >= 0:
            gpu.hot.decref(gpu.bases[g])
    evicted_n = gpu.hot.evict_unreferenced()
    assert evicted_n == evicted_o
    cs, hs = gpu.cold.state(), gpu.hot.state()
    oc, oh = sim.cold.state(), sim.hot.state()
    assert cs == oc and hs == oh, "final allocator state differs from the oracle"
    assert all(r == 0 for r in cs["ref"]) and len(cs["free"]) == wl.num_cold_pages and cs["seqs"] == {}
    assert hs["slabs"] == []
    return choices_seen


def small_workload(seed=21):
    return W.make_custom(batch=10, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16",
                         group_prefix_len=[300, 45, 1100], group_of=[0, 0, 1, 1, 2, 2, -1, 0, 2, 1],
                         suffix_len=[40, 3, 17, 100, 1, 64, 33, 250, 16, 90], seed=seed, extra_steps=40)


@pytest.mark.parametrize("P", [1, 16])
def test_multistep_small_all_rows(P):
    note(f"[gpu] multistep small P={P}")
    run(small_workload(), P, lambda s, n, rng: None)


@pytest.mark.parametrize("P", [1, 16])
def test_multistep_small_fused_appends(P):
    # forks, releases and copy-on-write with the appends fused into the step
    note(f"[gpu] multistep small fused P={P}")
    run(small_workload(), P, lambda s, n, rng: None, fused=True)


C4_FULL_STEPS = (0, 8, 9, 24, 25, 31)   # first step, the forks and the step after, the releases and after, last


@pytest.mark.timeout(900)
@pytest.mark.parametrize("P", [1, 16])
def test_multistep_c4(P):
    # The full heterogeneous multi-agent run at page size 1 and 16 (copy-on-write
    # after the forks): every row at the first step, around the forks and the
    # releases and at the last step; two sampled rows at the other steps; the
    # copy-on-write invariant on the device after every step from the forks on.
    wl = W.make_workload(W.CONFIGS["C4"], page_size=P)
    note(f"[gpu] multistep C4: B={wl.batch} groups={len(wl.group_prefix_len)} P={P}")
    seen = run(wl, P, lambda s, n, rng: None if s in C4_FULL_STEPS
               else sorted(rng.choice(n, size=2, replace=False).tolist()))
    # per-group mode takes the cascade for the long shared prefixes
    assert any(all(c) for c in seen[A.SPKV_MODE_PER_GROUP])
