"""Pins for the oracle's multi-step driver (CPU).

``MultiStepSim`` runs the heterogeneous multi-agent schedule of the GraniKV
paper (Section 4.5, Appendix B.8b: several prefix groups, forks, releases)
through the oracle allocators, using the "Paged KV cache" page's fork and
release (Code section).  Here it runs a tiny schedule and every step is
checked against what the pages fix, independently of the driver's own
bookkeeping:
  * a page's refcount equals the number of live block tables holding it, and
    the free stack is exactly the unreferenced pages (no duplicates);
  * a HOT slab's refcount equals the live requests of its group;
  * each live request's logical history (COLD length and K/V rows) equals the
    one built here from the draws: its drawn suffix, then one new token per
    step it was live; a fork child starts from its parent's history;
  * the forks at ``fork_step`` fork the first request of each group, the
    releases at ``release_step`` retire exactly those parents;
  * teardown returns every reference to zero and both pools to full;
  * ``reference`` equals the (separately pinned) flat oracle on a workload
    assembled here from the expected histories.
Each check names the mistake it catches.
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from oracle.attention import decode_reference
from oracle.driver import MultiStepSim

FORK, RELEASE, STEPS = 2, 4, 6


def tiny(P):
    return W.make_custom(batch=6, num_q_heads=4, num_kv_heads=2, head_dim=8, dtype="f32",
                         group_prefix_len=[5, 7], group_of=[0, 0, 1, 1, -1, 0],
                         suffix_len=[3, 1, 4, 2, 5, 1], page_size=P, seed=3, extra_steps=8)


def live_after(sim, s):
    """Live ids the step will attend (forks add, releases remove), from the schedule."""
    live = set(sim.live)
    if s == FORK:
        firsts = {}
        for b in sorted(live):
            g = sim.group_of[b]
            if g >= 0:
                firsts.setdefault(g, b)
        live |= {max(sim.group_of) + 1 + i for i in range(len(firsts))}
    if s == RELEASE:
        live -= set(sim.fork_parents)
    return len(live)


def check_refcounts(sim):
    # Catches: fork not sharing (or double-counting) pages, release skipping a
    # page, CoW not dropping the old page's reference.
    pool = sim.cold
    held = np.zeros(pool.num_pages, dtype=np.int64)
    for sid, s in pool.seqs.items():
        if s.live:
            for p in set(s.table):
                held[p] += 1
    assert list(held) == pool.ref
    assert len(pool.free) == len(set(pool.free))
    assert sorted(pool.free) == [p for p in range(pool.num_pages) if pool.ref[p] == 0]


def check_hot_refs(sim):
    # Catches: a fork that does not incref the group's slab, or a release that
    # does not decref it.
    for g, base in enumerate(sim.bases):
        members = sum(1 for b in sim.live if sim.group_of[b] == g)
        assert sim.hot.slabs[base].ref == members


def run_and_check(P, sim_cls=MultiStepSim):
    wl = tiny(P)
    B = wl.batch
    sim = sim_cls(wl, page_size=P, fork_step=FORK, release_step=RELEASE)
    # Expected histories, built from the draws alone.
    hist = {b: [wl.suffix_kv(b)[0][:-1], wl.suffix_kv(b)[1][:-1]] for b in range(B)}
    hist = {b: (list(k), list(v)) for b, (k, v) in hist.items()}
    check_refcounts(sim)
    check_hot_refs(sim)
    cows_seen = 0
    for s in range(STEPS):
        n_live = live_after(sim, s)
        dr = W.step_draws(wl.cfg, s, n_live)
        before_live = sorted(sim.live)
        rec = sim.step(dr.k_new, dr.v_new)
        cows_seen += len(rec.cows)
        if s == FORK:
            # Catches: forking the wrong member, or children with the wrong ids.
            firsts = {}
            for b in before_live:
                if sim.group_of[b] >= 0:
                    firsts.setdefault(sim.group_of[b], b)
            assert rec.forked == {firsts[g]: B + i for i, g in enumerate(sorted(firsts))}
            for parent, child in rec.forked.items():
                assert sim.group_of[child] == sim.group_of[parent]
                hist[child] = (list(hist[parent][0]), list(hist[parent][1]))
        else:
            assert rec.forked == {}
        if s == RELEASE:
            # Catches: releasing children instead of parents, or leaving a parent live.
            assert rec.released == sorted(sim.fork_parents)
            for p in rec.released:
                assert p not in rec.live and not sim.cold.seqs[p].live
        else:
            assert rec.released == []
        assert rec.live == sorted(rec.live) and len(rec.live) == n_live
        for i, b in enumerate(rec.live):
            hist[b][0].append(dr.k_new[i])
            hist[b][1].append(dr.v_new[i])
        check_refcounts(sim)
        check_hot_refs(sim)
        for b in rec.live:
            # Catches: a history shared by reference between parent and child
            # (the parent's later tokens would leak into the child), a dropped
            # or doubled token, a COLD length out of step with the history.
            k = np.concatenate(sim.hist_k[b], axis=0)
            v = np.concatenate(sim.hist_v[b], axis=0)
            np.testing.assert_array_equal(k, np.stack(hist[b][0]))
            np.testing.assert_array_equal(v, np.stack(hist[b][1]))
            assert sim.cold.length(b) == len(hist[b][0]) == rec.lens[b]
            assert len(rec.tables[b]) == -(-rec.lens[b] // P)
        # reference(): the flat oracle over a workload assembled from the
        # expected histories.  Catches: the wrong q row, the wrong group's
        # prefix, or a history that is not the request's.
        gof = np.array([sim.group_of[b] for b in rec.live], dtype=np.int32)
        sk = np.concatenate([np.stack(hist[b][0]) for b in rec.live])
        sv = np.concatenate([np.stack(hist[b][1]) for b in rec.live])
        ls = np.array([len(hist[b][0]) for b in rec.live], dtype=np.int64)
        wl_s = dataclasses.replace(wl, group_of=gof, suffix_len=ls, suffix_k=sk, suffix_v=sv, q=dr.q,
                                   suffix_offsets=None, cfg=dataclasses.replace(wl.cfg, batch=len(rec.live)))
        wl_s.__post_init__()
        ro, rl = decode_reference(wl_s)
        so, sl = sim.reference(rec.live, dr.q)
        np.testing.assert_allclose(so, ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(sl, rl, rtol=0, atol=1e-12)
        go, gl = sim.reference_grouped(rec.live, dr.q)
        np.testing.assert_allclose(go, ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(gl, rl, rtol=0, atol=1e-12)
    if P > 1:
        assert cows_seen > 0            # the forks' shared partial pages were copied on write
    # Teardown (spec invariant: refcounts return to zero after release).
    # Catches: a leaked reference, a slab never released, a page lost from the stack.
    evicted = sim.finish()
    assert evicted == len(sim.bases)
    assert sim.cold.ref == [0] * sim.cold.num_pages and sim.cold.num_free() == sim.cold.num_pages
    assert sim.hot.slabs == {} and sim.hot.free == [(0, sim.hot.capacity)]


@pytest.mark.parametrize("P", [1, 4])
def test_multistep_schedule_against_the_pages(P):
    run_and_check(P)


class AliasingSim(MultiStepSim):
    """A planted mistake (CPU only): fork children alias the parent's history list."""

    def step(self, k_new, v_new):
        if self.step_index == self.fork_step:
            rec = super().step(k_new, v_new)
            for parent, child in rec.forked.items():
                self.hist_k[child] = self.hist_k[parent]
            return rec
        return super().step(k_new, v_new)


class NoHotIncrefSim(MultiStepSim):
    """A planted mistake (CPU only): the fork forgets the group's slab reference."""

    def step(self, k_new, v_new):
        forking = self.step_index == self.fork_step
        rec = super().step(k_new, v_new)
        if forking:
            for parent in rec.forked:
                self.hot.decref(self.bases[self.group_of[parent]])
        return rec


@pytest.mark.parametrize("planted", [AliasingSim, NoHotIncrefSim])
def test_multistep_checks_catch_planted_mistakes(planted):
    with pytest.raises(AssertionError):
        run_and_check(1, planted)
