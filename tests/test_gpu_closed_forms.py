"""Closed-form properties of decode attention checked on the HIP path at
sizes where a dropped, duplicated or misplaced token would show exactly
(needs an MI355X).  Each case follows from the definition of softmax
attention (GraniKV paper, Sections 2.1/2.3): zero queries weight every token
equally; constant values pass through; a key far above the rest takes all
the weight.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle.attention import widen
from shared_prefix_paged_amd import runtime as R
from hip_setup import setup_single_step

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def base_workload(seed=31, lp=(1500, 300), ls=None, dtype="bf16", d=128, hq=16, hkv=4):
    ls = ls if ls is not None else [700, 3, 1, 257, 64, 2000, 33, 130]
    B = len(ls)
    gof = [0, 0, 1, 0, 1, -1, 0, 1][:B]
    return W.make_custom(batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                         group_prefix_len=list(lp), group_of=gof, suffix_len=ls, seed=seed)


def run_both(wl):
    st = setup_single_step(wl)
    ws = R.workspace(st.batch)
    res = []
    for fn in (R.cascade_decode, R.dense_decode):
        out, lse = fn(st.batch, st.pools, ws)
        torch.cuda.synchronize()
        res.append((fn.__name__, out.cpu().double().numpy(), lse.cpu().double().numpy()))
    return res


def ctx_len(wl, b):
    return wl.prefix_len_of(b) + int(wl.suffix_len[b])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_query_mean_and_log_count(dtype):
    wl = base_workload(dtype=dtype)
    wl.q[:] = 0
    note(f"[gpu] zero query {dtype}")
    G = wl.cfg.group_size
    for name, o, l in run_both(wl):
        for b in range(wl.batch):
            g = int(wl.group_of[b])
            sk, sv = wl.suffix_kv(b)
            parts = [widen(sv, dtype)] + ([widen(wl.prefix_v[g], dtype)] if g >= 0 else [])
            mean = np.concatenate(parts, axis=0).mean(axis=0)          # [Hkv, d]
            for j in range(wl.cfg.num_q_heads):
                np.testing.assert_allclose(o[b, j], mean[j // G], atol=2e-6, err_msg=f"{name} b={b} j={j}")
            np.testing.assert_allclose(l[b], math.log(ctx_len(wl, b)), atol=2e-5, err_msg=name)


def test_constant_values():
    wl = base_workload()
    c = W.bf16_bits_from_f32(np.float32([-0.8125]))[0]
    for arr in wl.prefix_v + [wl.suffix_v]:
        arr[:] = c
    note("[gpu] constant V")
    for name, o, l in run_both(wl):
        np.testing.assert_allclose(o, -0.8125, atol=1e-6, err_msg=name)


def test_counting_prefix_vs_suffix_tokens():
    wl = base_workload()
    wl.q[:] = 0
    one = W.bf16_bits_from_f32(np.float32([1.0]))[0]
    for arr in wl.prefix_v:
        arr[:] = 0
        arr[:, :, 0] = one
    wl.suffix_v[:] = 0
    wl.suffix_v[:, :, 0] = one
    wl.suffix_v[:, :, 1] = one
    note("[gpu] counting")
    for name, o, l in run_both(wl):
        for b in range(wl.batch):
            np.testing.assert_allclose(o[b, :, 0], 1.0, atol=1e-6)
            np.testing.assert_allclose(o[b, :, 1], int(wl.suffix_len[b]) / ctx_len(wl, b), atol=2e-6,
                                       err_msg=f"{name} b={b}")


@pytest.mark.parametrize("where", ["prefix", "suffix"])
def test_needle_key_takes_the_weight(where):
    wl = base_workload(seed=33)
    G = wl.cfg.group_size
    rng = np.random.default_rng(1)
    chosen = {}
    for b in range(wl.batch):
        g = int(wl.group_of[b])
        if where == "prefix" and g < 0:
            continue
        q = widen(wl.q[b], "bf16")
        for h in range(wl.cfg.num_kv_heads):
            # needle for query head h*G of request b; 8*q is exact in bf16
            k_needle = W.bf16_bits_from_f32((8.0 * q[h * G]).astype(np.float32))
            if where == "prefix":
                t = int(rng.integers(0, int(wl.group_prefix_len[g])))
                wl.prefix_k[g][t, h] = k_needle
                chosen[(b, h)] = widen(wl.prefix_v[g][t, h], "bf16")
            else:
                sk, sv = wl.suffix_kv(b)
                t = int(rng.integers(0, sk.shape[0]))
                row = int(wl.suffix_offsets[b]) + t
                wl.suffix_k[row, h] = k_needle
                chosen[(b, h)] = widen(wl.suffix_v[row, h], "bf16")
        if where == "prefix":
            break   # one request per prefix group keeps the needles unambiguous
    note(f"[gpu] needle in {where}")
    for name, o, l in run_both(wl):
        for (b, h), v in chosen.items():
            np.testing.assert_allclose(o[b, h * G], v, atol=1e-5, err_msg=f"{name} b={b} h={h}")
