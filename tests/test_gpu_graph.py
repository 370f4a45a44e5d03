"""The decode step as a HIP graph (needs an MI355X): spkv_graph_decode_step_append
against the direct spkv_decode_step_append over several steps from identical
states, bit for bit (outputs, LSE, pools, device block tables and lengths).
Direct (eager) calls run between the graph's replays and every replay is
checked, so a node that replays stale arguments, or work of the graph that
does not repeat, fails."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from shared_prefix_paged_amd import runtime as R
from shared_prefix_paged_amd import _abi as A
from hip_setup import setup_single_step, to_device, pool_bytes

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("P", [1, 16])
def test_graph_step_matches_direct_step(P):
    wl = W.make_custom(batch=20, num_q_heads=16, num_kv_heads=4, head_dim=128, dtype="bf16",
                       group_prefix_len=[700, 90], group_of=[0] * 12 + [1] * 6 + [-1] * 2,
                       suffix_len=[int(x) for x in np.random.default_rng(70).integers(1, 300, 20)], seed=70,
                       page_size=P)
    cfg = wl.cfg
    B, hkv, d = wl.batch, cfg.num_kv_heads, cfg.head_dim
    steps = 6
    mb = (int(wl.suffix_len.max()) + steps + P - 1) // P + 1
    states = [setup_single_step(wl, max_blocks=mb) for _ in range(2)]
    graph = R.StepGraph()
    params = R.default_params(A.SPKV_MODE_PER_GROUP)
    insts = []
    for step in range(steps):
        dr = W.step_draws(cfg, step + 1, B)
        k, v, q = (to_device(x, "bf16") for x in (dr.k_new, dr.v_new, dr.q))
        res = []
        for j, st in enumerate(states):
            slots, cows = st.cold.append_batch(np.asarray(st.seqs, np.int32))
            if cows:
                R.copy_blocks(torch.tensor(cows, dtype=torch.int32, device="cuda"), st.pools.k_cold,
                              st.pools.v_cold, st.cold.num_pages, P, hkv, d)
            st.batch.lens_h += 1
            st.batch.struct.q = q.data_ptr()
            ws = R.workspace(st.batch)
            if j == 0:
                out, lse, _ = R.decode_step_append(st.batch, st.pools, params, ws, k, v, slots)
            else:
                out, lse, _, inst = graph.decode_step_append(st.batch, st.pools, params, ws, k, v, slots)
                insts.append(inst)
            torch.cuda.synchronize()
            res.append((out.clone(), lse.clone()))
        note(f"[gpu] graph P={P} step {step}: instantiated={insts[-1]}")
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1]), f"step {step}"
        for a, b in ((states[0].pools.k_cold, states[1].pools.k_cold), (states[0].pools.v_cold, states[1].pools.v_cold)):
            np.testing.assert_array_equal(pool_bytes(a), pool_bytes(b))
        assert torch.equal(states[0].batch.tables, states[1].batch.tables)
        assert torch.equal(states[0].batch.lens, states[1].batch.lens)
    assert insts[0]                               # the first call instantiates
    assert not all(insts[1:]) or len(insts) == 1  # later steps update the graph in place at least once
    graph.close()
