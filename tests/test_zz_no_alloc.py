"""spkv_decode_step_append_noalloc against spkv_decode_step_append (needs an
MI355X): the entry point without a workspace, for callers that cannot
allocate, keeps its partial states in the library's static scratch.  Two
calls in a row, the second on a smaller batch (the scratch keeps the first
call's contents), each equal bit for bit to the workspace entry point's result
on the same inputs and within the oracle's tolerance; pools, block tables and
lengths advance identically."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle.attention import decode_reference
from shared_prefix_paged_amd import runtime as R
from shared_prefix_paged_amd import _abi as A
from hip_setup import setup_single_step, errors, to_device

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE, TOL_REL = 2e-3, 1e-3, 1e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def workloads():
    big = W.make_custom(batch=48, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                        group_prefix_len=[2000, 333], group_of=[0] * 30 + [1] * 14 + [-1] * 4,
                        suffix_len=[int(x) for x in np.random.default_rng(40).integers(1, 1500, 48)], seed=40)
    small = W.make_custom(batch=5, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="bf16",
                          group_prefix_len=[70], group_of=[0, 0, -1, 0, 0], suffix_len=[3, 1, 40, 17, 9], seed=41)
    return [("48 requests, d=128", big), ("5 requests, d=64", small)]


def one_call(fn, st, wl, ws=None):
    off = wl.suffix_offsets
    k_new = to_device(wl.suffix_k[off[1:] - 1], wl.cfg.dtype)
    v_new = to_device(wl.suffix_v[off[1:] - 1], wl.cfg.dtype)
    st.batch.lens -= 1                      # the device view before the step's append
    params = R.default_params(A.SPKV_MODE_PER_GROUP)
    if ws is None:
        out, lse, _ = fn(st.batch, st.pools, params, k_new, v_new, st.step_slots)
    else:
        out, lse, _ = fn(st.batch, st.pools, params, ws, k_new, v_new, st.step_slots)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.batch.lens.cpu().numpy(), st.lens)
    np.testing.assert_array_equal(st.batch.tables.cpu().numpy().reshape(st.tables.shape), st.tables)
    return out.clone(), lse.clone()


def test_noalloc_matches_workspace_entry_point_twice():
    for name, wl in workloads():
        note(f"[gpu] noalloc: {name}")
        ref_o, ref_l = decode_reference(wl)
        st = setup_single_step(wl)
        ws = R.workspace(st.batch)
        o_ws, l_ws = one_call(R.decode_step_append, st, wl, ws)
        o_na, l_na = one_call(R.decode_step_append_noalloc, st, wl)
        e_o, e_l, rel = errors(o_na, l_na, ref_o, ref_l)
        note(f"    max_abs={e_o:.3e} lse={e_l:.3e} rel={rel:.3e}")
        assert e_o <= TOL_O and e_l <= TOL_LSE and rel <= TOL_REL
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
