"""Reference decode attention in float64 (oracle; test infrastructure only).

What the method computes (GraniKV paper, Sections 2.1 and 2.3; "Paged KV
cache" page, "How it works" step 3): for request b and query head j, whose KV
head is h = floor(j / G) with G the GQA group size, over the logical
concatenation of the request's prefix tokens (Lp of them, 0 when it has no
HOT prefix) and its suffix tokens (Ls, which include the token being decoded):

    s_t   = scale * <q_bj, k_th>
    O_bj  = sum_t exp(s_t - m) v_th / sum_t exp(s_t - m),   m = max_t s_t
    LSE_bj = m + ln sum_t exp(s_t - m)                        (natural log)

Cascade attention (paper, Section 2.3) reaches the same result in three parts:
the prefix part, the suffix part, and the log-sum-exp merge of its Eq. (1),
read as a weighted mean of the two normalised partial outputs with weights
exp(l_p - m) and exp(l_s - m), m = max(l_p, l_s).  An empty part has
LSE = -inf and weight 0 (both empty: O = 0, LSE = -inf).

All arithmetic is float64 on the exact input values (bf16 bit patterns are
widened exactly).  A matrix product from numpy serves as a step; nothing is
blocked, fused or reordered beyond the definition.

``attend_shared_prefix`` and ``decode_reference_grouped`` compute the same
definition for many rows that share one prefix: the prefix scores of all rows
come from one matrix product, each row's suffix scores from its own tokens,
and every row still takes one max and one normaliser over all of its tokens.
They exist so that every row of a full-size configuration can be checked in
seconds (the prefix is widened to float64 once per group, not per request).

Pinned by ``tests/test_oracle_attention.py``: closed forms (Q = 0, constant V,
one token, token counting, a needle key), 50-digit brute force on tiny inputs,
cascade = flat, page-size and slot-permutation invariance, merge identities;
the grouped forms by the same closed forms and by agreement with the per-row
form on drawn workloads.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")


def widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16) or float32 data."""
    if dtype == "bf16":
        a = np.asarray(arr, dtype=np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def attend(q_rows: np.ndarray, k_parts: Sequence[np.ndarray], v_parts: Sequence[np.ndarray],
           scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of query rows over the concatenation of token parts.

    q_rows [R, d]; each k/v part [N_i, d] (float64).  Returns O [R, d], LSE [R].
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, d = q_rows.shape
    scores = [scale * (k @ q_rows.T) for k in k_parts]          # each [N_i, R]
    n_total = sum(s.shape[0] for s in scores)
    if n_total == 0:
        return np.zeros((R, d)), np.full(R, NEG_INF)
    m = np.max(np.concatenate(scores, axis=0), axis=0)           # [R]
    num = np.zeros((R, d))
    den = np.zeros(R)
    for s, v in zip(scores, v_parts):
        if s.shape[0] == 0:
            continue
        e = np.exp(s - m)                                        # [N_i, R]
        num += e.T @ v
        den += e.sum(axis=0)
    return num / den[:, None], m + np.log(den)


def attend_shared_prefix(q_rows: np.ndarray, prefix_k, prefix_v, suffix_parts, scale: float):
    """Rows that share one prefix, each with its own suffix tokens.

    q_rows [R, d]; prefix_k / prefix_v [Lp, d] or None; suffix_parts is a list
    of (row slice, k [Ls, d], v [Ls, d]) covering every row once (float64).
    Row r attends to the prefix tokens followed by its own suffix tokens.
    Returns O [R, d], LSE [R].
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R, d = q_rows.shape
    m = np.full(R, NEG_INF)
    sp = None
    if prefix_k is not None and prefix_k.shape[0] > 0:
        sp = scale * (q_rows @ prefix_k.T)                       # [R, Lp]
        m = np.max(sp, axis=1)
    ss = []
    for rows, k, v in suffix_parts:
        s = scale * (q_rows[rows] @ k.T)                         # [r, Ls]
        ss.append(s)
        if s.shape[1]:
            m[rows] = np.maximum(m[rows], np.max(s, axis=1))
    empty = np.isneginf(m)
    m_use = np.where(empty, 0.0, m)
    num = np.zeros((R, d))
    den = np.zeros(R)
    if sp is not None:
        e = np.exp(sp - m_use[:, None])
        num += e @ prefix_v
        den += e.sum(axis=1)
    for (rows, k, v), s in zip(suffix_parts, ss):
        if s.shape[1] == 0:
            continue
        e = np.exp(s - m_use[rows][:, None])
        num[rows] += e @ v
        den[rows] += e.sum(axis=1)
    den_use = np.where(empty, 1.0, den)
    out = np.where(empty[:, None], 0.0, num / den_use[:, None])
    lse = np.where(empty, NEG_INF, m_use + np.log(den_use))
    return out, lse


def decode_reference_grouped(wl, scale: float = None):
    """Every row of a drawn workload, group by group (same values as decode_reference)."""
    cfg = wl.cfg
    dt, G = cfg.dtype, cfg.group_size
    hkv = cfg.num_kv_heads
    scale = (1.0 / np.sqrt(cfg.head_dim)) if scale is None else scale
    B, Hq, d = wl.q.shape
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), NEG_INF)
    groups = sorted(set(int(g) for g in wl.group_of))
    for g in groups:
        members = [int(b) for b in np.flatnonzero(wl.group_of == g)]
        pk = widen(wl.prefix_k[g], dt) if g >= 0 else None
        pv = widen(wl.prefix_v[g], dt) if g >= 0 else None
        suffix = [tuple(widen(x, dt) for x in wl.suffix_kv(b)) for b in members]
        for h in range(hkv):
            q = np.concatenate([widen(wl.q[b, h * G:(h + 1) * G], dt) for b in members])
            parts = [(slice(i * G, (i + 1) * G), sk[:, h], sv[:, h]) for i, (sk, sv) in enumerate(suffix)]
            o, l = attend_shared_prefix(q, None if pk is None else pk[:, h], None if pv is None else pv[:, h],
                                        parts, scale)
            for i, b in enumerate(members):
                out[b, h * G:(h + 1) * G] = o[i * G:(i + 1) * G]
                lse[b, h * G:(h + 1) * G] = l[i * G:(i + 1) * G]
    return out, lse


def merge(o_a: np.ndarray, lse_a: np.ndarray, o_b: np.ndarray, lse_b: np.ndarray):
    """Eq. (1): combine two normalised partial states row by row."""
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - m_safe))
    wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - m_safe))
    w = wa + wb
    w_safe = np.where(empty, 1.0, w)
    o = (wa[..., None] * o_a + wb[..., None] * o_b) / w_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, NEG_INF, m_safe + np.log(w_safe))
    return o, lse


def decode_request(q_b: np.ndarray, prefix_k, prefix_v, suffix_k, suffix_v, scale: float, group: int):
    """One request, all query heads.  q_b [Hq, d]; prefix/suffix K/V [N, Hkv, d] (float64)."""
    Hq, d = q_b.shape
    hkv = suffix_k.shape[1] if suffix_k is not None and suffix_k.ndim == 3 else prefix_k.shape[1]
    out = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    for h in range(hkv):
        rows = slice(h * group, (h + 1) * group)
        ks, vs = [], []
        if prefix_k is not None:
            ks.append(prefix_k[:, h, :])
            vs.append(prefix_v[:, h, :])
        ks.append(suffix_k[:, h, :])
        vs.append(suffix_v[:, h, :])
        out[rows], lse[rows] = attend(q_b[rows], ks, vs, scale)
    return out, lse


def decode_reference(wl, rows: Sequence[int] = None, scale: float = None):
    """Flat reference for a drawn workload: O [B, Hq, d] and LSE [B, Hq] (float64).

    ``rows`` restricts the computation to some requests (others stay zero)."""
    cfg = wl.cfg
    dt, G = cfg.dtype, cfg.group_size
    scale = (1.0 / np.sqrt(cfg.head_dim)) if scale is None else scale
    B, Hq, d = wl.q.shape
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), NEG_INF)
    pk = [widen(k, dt) for k in wl.prefix_k]
    pv = [widen(v, dt) for v in wl.prefix_v]
    for b in (range(B) if rows is None else rows):
        g = int(wl.group_of[b])
        sk, sv = wl.suffix_kv(b)
        out[b], lse[b] = decode_request(widen(wl.q[b], dt),
                                        pk[g] if g >= 0 else None, pv[g] if g >= 0 else None,
                                        widen(sk, dt), widen(sv, dt), scale, G)
    return out, lse


def cascade_reference(wl, scale: float = None):
    """Prefix part, suffix part and Eq. (1) merge, computed separately (float64)."""
    cfg = wl.cfg
    dt, G = cfg.dtype, cfg.group_size
    scale = (1.0 / np.sqrt(cfg.head_dim)) if scale is None else scale
    B, Hq, d = wl.q.shape
    hkv = cfg.num_kv_heads
    o_p = np.zeros((B, Hq, d)); l_p = np.full((B, Hq), NEG_INF)
    o_s = np.zeros((B, Hq, d)); l_s = np.full((B, Hq), NEG_INF)
    for b in range(B):
        g = int(wl.group_of[b])
        q = widen(wl.q[b], dt)
        sk, sv = wl.suffix_kv(b)
        sk, sv = widen(sk, dt), widen(sv, dt)
        for h in range(hkv):
            r = slice(h * G, (h + 1) * G)
            if g >= 0:
                o_p[b, r], l_p[b, r] = attend(q[r], [widen(wl.prefix_k[g][:, h], dt)],
                                              [widen(wl.prefix_v[g][:, h], dt)], scale)
            o_s[b, r], l_s[b, r] = attend(q[r], [sk[:, h]], [sv[:, h]], scale)
    o, l = merge(o_p, l_p, o_s, l_s)
    return o, l, (o_p, l_p, o_s, l_s)
