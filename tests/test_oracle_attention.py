"""Pins for the oracle's attention (CPU).

Closed forms that a dropped term, wrong sign, wrong scale, transposed operand
or wrong GQA index would break; 50-digit brute force on tiny inputs; the
method's invariants (cascade + Eq. (1) merge equals flat attention, page size
and slot permutation do not change the result, merge identities).
"""
import math

import mpmath
import numpy as np
import pytest

import workloads as W
from oracle.attention import attend, merge, decode_reference, cascade_reference, widen, NEG_INF, attend_shared_prefix, decode_reference_grouped
from oracle.driver import run_single_step, paged_reference


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --- closed forms -----------------------------------------------------------

def test_zero_query_gives_mean_and_log_count():
    k1, k2 = rnd((37, 16), 1), rnd((5, 16), 2)
    v1, v2 = rnd((37, 16), 3), rnd((5, 16), 4)
    o, l = attend(np.zeros((3, 16)), [k1, k2], [v1, v2], 0.25)
    mean = np.concatenate([v1, v2]).mean(axis=0)
    np.testing.assert_allclose(o, np.tile(mean, (3, 1)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, math.log(42), rtol=0, atol=1e-14)


def test_constant_values_pass_through():
    q, k = rnd((4, 8), 5), rnd((50, 8), 6)
    o, _ = attend(q, [k[:20], k[20:]], [np.full((20, 8), -1.75), np.full((30, 8), -1.75)], 0.3)
    np.testing.assert_allclose(o, -1.75, rtol=0, atol=1e-14)


def test_single_token():
    q, k, v = rnd((2, 8), 7), rnd((1, 8), 8), rnd((1, 8), 9)
    o, l = attend(q, [k], [v], 0.5)
    np.testing.assert_allclose(o, np.tile(v[0], (2, 1)), atol=1e-15)
    np.testing.assert_allclose(l, 0.5 * (q @ k[0]), atol=1e-14)


def test_two_token_weights_pin_scale_and_sign():
    # q = a e0, k1 = e0, k2 = 0 -> s1 = scale * a, s2 = 0
    a, scale = 3.0, 0.125
    q = np.zeros((1, 4)); q[0, 0] = a
    k = np.zeros((2, 4)); k[0, 0] = 1.0
    v = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    o, l = attend(q, [k], [v], scale)
    w1 = math.exp(scale * a) / (math.exp(scale * a) + 1.0)
    np.testing.assert_allclose(o[0], [w1, 1 - w1, 0, 0], atol=1e-15)
    assert abs(l[0] - math.log(math.exp(scale * a) + 1.0)) < 1e-15


def test_counting_prefix_and_suffix_tokens():
    lp, ls, d = 300, 17, 8
    vp = np.zeros((lp, d)); vp[:, 0] = 1
    vs = np.zeros((ls, d)); vs[:, 0] = 1; vs[:, 1] = 1
    o, l = attend(np.zeros((4, d)), [rnd((lp, d), 1), rnd((ls, d), 2)], [vp, vs], 0.3)
    np.testing.assert_allclose(o[:, 0], 1.0, atol=1e-14)
    np.testing.assert_allclose(o[:, 1], ls / (lp + ls), atol=1e-14)
    np.testing.assert_allclose(l, math.log(lp + ls), atol=1e-13)


def test_needle_token_dominates():
    d, n = 64, 500
    q = rnd((1, d), 3)
    k = rnd((n, d), 4)
    v = rnd((n, d), 5)
    k[123] = 8 * q[0]
    o, _ = attend(q, [k[:200], k[200:]], [v[:200], v[200:]], 1 / 8)
    np.testing.assert_allclose(o[0], v[123], atol=1e-12)


def test_empty_gives_identity_state():
    o, l = attend(rnd((2, 4), 1), [np.zeros((0, 4))], [np.zeros((0, 4))], 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_gqa_head_mapping_is_floor_division():
    """Hq = 4, Hkv = 2: query heads 0,1 read KV head 0; heads 2,3 read KV head 1."""
    wl = W.make_custom(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=8, dtype="f32",
                       group_prefix_len=[6], group_of=[0], suffix_len=[3], seed=1)
    wl.q[:] = 0
    for arr in (wl.prefix_v[0], wl.suffix_v):
        arr[:, 0, :] = 1.0
        arr[:, 1, :] = 2.0
    o, _ = decode_reference(wl)
    np.testing.assert_allclose(o[0, :, 0], [1, 1, 2, 2], atol=1e-15)


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xC000, 0x3E00, 0x0001, 0x7F7F], dtype=np.uint16)
    vals = widen(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 0.125
    assert vals[3] == 2.0 ** -133
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127


# --- brute force at 50 digits --------------------------------------------------

def mp_attend(q, k, v, scale):
    mpmath.mp.dps = 50
    n, d = k.shape
    out, lses = [], []
    for r in range(q.shape[0]):
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[r, c]) * mpmath.mpf(k[t, c]) for c in range(d))
             for t in range(n)]
        z = mpmath.fsum(mpmath.e ** x for x in s)
        o = [mpmath.fsum(mpmath.e ** s[t] * mpmath.mpf(v[t, c]) for t in range(n)) / z for c in range(d)]
        out.append([float(x) for x in o])
        lses.append(float(mpmath.log(z)))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 9)); d = int(rng.integers(1, 5)); r = int(rng.integers(1, 4))
    q, k, v = rng.standard_normal((r, d)) * 2, rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d))
    split = int(rng.integers(0, n + 1))
    o, l = attend(q, [k[:split], k[split:]], [v[:split], v[split:]], 0.7)
    o2, l2 = mp_attend(q, k, v, 0.7)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, l2, rtol=0, atol=1e-14)


# --- merge (Eq. 1) ----------------------------------------------------------------

def test_merge_identities():
    rng = np.random.default_rng(3)
    o = [rng.standard_normal((5, 7)) for _ in range(3)]
    l = [rng.standard_normal(5) * 4 for _ in range(3)]
    ab = merge(o[0], l[0], o[1], l[1]); ba = merge(o[1], l[1], o[0], l[0])
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-15); np.testing.assert_allclose(ab[1], ba[1], atol=1e-15)
    left = merge(*merge(o[0], l[0], o[1], l[1]), o[2], l[2])
    right = merge(o[0], l[0], *merge(o[1], l[1], o[2], l[2]))
    np.testing.assert_allclose(left[0], right[0], atol=1e-15); np.testing.assert_allclose(left[1], right[1], atol=1e-14)
    ident = merge(o[0], l[0], np.zeros((5, 7)), np.full(5, NEG_INF))
    np.testing.assert_array_equal(ident[0], o[0]); np.testing.assert_allclose(ident[1], l[0], atol=0)
    both = merge(np.zeros((5, 7)), np.full(5, NEG_INF), np.zeros((5, 7)), np.full(5, NEG_INF))
    assert np.all(both[0] == 0) and np.all(np.isneginf(both[1]))


def test_merge_of_split_equals_whole():
    q, k, v = rnd((3, 16), 1), rnd((90, 16), 2), rnd((90, 16), 3)
    whole = attend(q, [k], [v], 0.25)
    a = attend(q, [k[:31]], [v[:31]], 0.25)
    b = attend(q, [k[31:]], [v[31:]], 0.25)
    m = merge(a[0], a[1], b[0], b[1])
    np.testing.assert_allclose(m[0], whole[0], atol=1e-14); np.testing.assert_allclose(m[1], whole[1], atol=1e-13)


# --- the method's invariants on drawn workloads -------------------------------------

def multi_group_workload(dtype="bf16", seed=9):
    return W.make_custom(batch=7, num_q_heads=8, num_kv_heads=2, head_dim=32, dtype=dtype,
                         group_prefix_len=[40, 17], group_of=[0, 0, 1, -1, 1, 0, 1],
                         suffix_len=[5, 1, 33, 9, 16, 17, 2], seed=seed)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cascade_equals_flat(dtype):
    wl = multi_group_workload(dtype)
    o, l = decode_reference(wl)
    oc, lc, _ = cascade_reference(wl)
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lc, l, rtol=0, atol=1e-12)


def test_c0_cascade_equals_flat():
    wl = W.make_workload(W.CONFIGS["C0"])
    o, l = decode_reference(wl)
    oc, lc, _ = cascade_reference(wl)
    np.testing.assert_allclose(oc, o, atol=1e-12); np.testing.assert_allclose(lc, l, atol=1e-12)


def test_page_size_and_slot_shuffle_invariance():
    wl1 = multi_group_workload()
    logical = decode_reference(wl1)
    outs = []
    for P in (1, 16):
        wl = W.make_custom(batch=7, num_q_heads=8, num_kv_heads=2, head_dim=32, dtype="bf16",
                           group_prefix_len=[40, 17], group_of=[0, 0, 1, -1, 1, 0, 1],
                           suffix_len=[5, 1, 33, 9, 16, 17, 2], seed=9, page_size=P)
        for fo in (None, "shuffled"):
            order = None if fo is None else list(np.random.default_rng(P).permutation(wl.num_cold_pages))
            st = run_single_step(wl, page_size=P, free_order=order)
            outs.append(paged_reference(st, wl))
    for o, l in outs:
        np.testing.assert_array_equal(o, outs[0][0])
        np.testing.assert_array_equal(l, outs[0][1])
    np.testing.assert_allclose(outs[0][0], logical[0], atol=1e-13)


# --- the grouped form (one prefix product for all rows of a group) ------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_grouped_equals_per_row(dtype):
    # Catches: a row taking another member's suffix, a max taken over the
    # prefix only, or the -1 group (no prefix) given a prefix.
    wl = multi_group_workload(dtype)
    o, l = decode_reference(wl)
    og, lg = decode_reference_grouped(wl)
    np.testing.assert_allclose(og, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lg, l, rtol=0, atol=1e-12)


def test_grouped_closed_forms():
    # Q = 0: every row's output is the mean of its prefix + suffix V rows and
    # its LSE is ln(Lp + Ls) (rows of one group have different suffixes).
    rng = np.random.default_rng(1)
    lp, d = 9, 4
    pk, pv = rng.standard_normal((lp, d)), rng.standard_normal((lp, d))
    suf = [(slice(0, 2), rng.standard_normal((3, d)), rng.standard_normal((3, d))),
           (slice(2, 3), rng.standard_normal((0, d)), rng.standard_normal((0, d))),
           (slice(3, 5), rng.standard_normal((7, d)), rng.standard_normal((7, d)))]
    o, l = attend_shared_prefix(np.zeros((5, d)), pk, pv, suf, 0.5)
    for rows, k, v in suf:
        allv = np.concatenate([pv, v])
        np.testing.assert_allclose(o[rows], np.broadcast_to(allv.mean(axis=0), o[rows].shape), atol=1e-14)
        np.testing.assert_allclose(l[rows], np.log(lp + k.shape[0]), atol=1e-14)
    # Needle in the suffix of row 3 only: key 8*q for a unit q dominates that row.
    q = np.zeros((5, d)); q[3, 0] = 1.0
    suf[2][1][4] = 8.0 * q[3]
    o, l = attend_shared_prefix(q, pk, pv, suf, 1.0)
    assert np.max(np.abs(o[3] - suf[2][2][4])) < 5e-2
    # No prefix and no suffix: the empty state.
    o, l = attend_shared_prefix(np.ones((1, d)), None, None, [(slice(0, 1), np.zeros((0, d)), np.zeros((0, d)))], 1.0)
    assert np.all(o == 0) and np.isneginf(l[0])
