"""Pins for the pages' cost formulas and the workload generator (CPU)."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from conftest import GOLDEN
from oracle import costmodel as cm
from oracle.pools import cold_slot, hot_offset


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def sig(x, digits):
    return float(f"{x:.{digits}g}")


def test_b11_byte_and_flop_model():
    g = load("granikv_b11_byte_model.json")
    B, lp, hq, hkv, d, e = g["batch"], g["prefix_len"], g["num_q_heads"], g["num_kv_heads"], g["head_dim"], g["elem_bytes"]
    n = g["printed_significant_digits"]
    assert sig(cm.paged_prefix_bytes(B, lp, hkv, d, e) / 1e9, n) == g["printed"]["paged_bytes_GB"]
    assert sig(cm.hot_prefix_bytes(lp, hkv, d, e) / 1e6, n) == g["printed"]["hot_bytes_MB"]
    assert sig(cm.prefix_flops(B, hq, lp, d) / 1e9, n) == g["printed"]["useful_GFLOP"]
    # exact values behind the printed figures
    assert cm.paged_prefix_bytes(B, lp, hkv, d, e) == 8_589_934_592
    assert cm.hot_prefix_bytes(lp, hkv, d, e) == 33_554_432
    assert cm.prefix_flops(B, hq, lp, d) == 34_359_738_368


def test_eq2_meff():
    g = load("granikv_eq2_meff.json")
    for c in g["cases"]:
        m = cm.m_eff(c["batch"], c["group_size"])
        assert m == c["m_eff"]
        assert (m >= g["m_sat_a100"]) == c["at_or_above_threshold"]


def test_bytes_per_token():
    g = load("paged_kv_bytes_per_token.json")
    for c in g["cases"]:
        per_tok = c["layers"] * cm.kv_bytes_per_token(c["kv_heads"], c["head_dim"], c["elem_bytes"])
        assert abs(per_tok - c["printed_bytes"]) <= g["relative_tolerance"] * c["printed_bytes"]


def test_slot_formula_picture():
    g = load("paged_kv_block_table_example.json")
    table = g["seq_a_table"]
    for lo, hi, blk in g["seq_a_token_blocks"]:
        for t in range(lo, hi + 1):
            assert cold_slot(table, t, g["block_size"]) == blk * 16 + t % 16


def test_hot_offset_hand_value():
    # base 100 tokens, Lp = 10, Hkv = 4, d = 8: head 2, token 3 starts at ((100*4 + 2*10) + 3) * 8
    assert hot_offset(100, 10, 4, 8, 3, 2) == 423 * 8
    # heads are disjoint, consecutive [Lp, d] blocks inside the slab [base*Hkv*d, (base+Lp)*Hkv*d)
    offs = sorted(hot_offset(100, 10, 4, 8, t, h) for h in range(4) for t in range(10))
    assert offs == list(range(100 * 4 * 8, 110 * 4 * 8, 8))


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -3.00390625, 65504.0]   # ties and a large value
    ours = W.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_workload_shapes_and_determinism():
    c0 = W.make_workload(W.CONFIGS["C0"])
    again = W.make_workload(W.CONFIGS["C0"])
    np.testing.assert_array_equal(c0.q, again.q)
    np.testing.assert_array_equal(c0.suffix_k, again.suffix_k)
    assert c0.q.shape == (4, 4, 64) and c0.q.dtype == np.float32
    assert c0.prefix_k[0].shape == (256, 1, 64)
    assert np.all((c0.suffix_len >= 1) & (c0.suffix_len <= 64))
    assert c0.suffix_k.shape[0] == c0.suffix_len.sum()
    assert sorted(c0.free_order) == list(range(c0.num_cold_pages))
    # page size changes only the free-order draw, not the tensors
    c0p = W.make_workload(W.CONFIGS["C0"], page_size=16)
    np.testing.assert_array_equal(c0p.suffix_k, c0.suffix_k)
    np.testing.assert_array_equal(c0p.q, c0.q)


def test_multi_prefix_workload_groups():
    cfg = W.CONFIGS["C4"]
    import dataclasses
    small = dataclasses.replace(cfg, prefix_range=(20, 40), suffix_range=(2, 9))
    wl = W.make_workload(small)
    assert wl.group_prefix_len.shape == (8,)
    assert np.all((wl.group_prefix_len >= 20) & (wl.group_prefix_len <= 40))
    assert list(np.bincount(wl.group_of)) == [16] * 8
    assert wl.hot_capacity == wl.group_prefix_len.sum()
