"""The pages' cost formulas (oracle; test infrastructure only).

GraniKV paper:
  * Eq. (2): the effective matmul M of a decode step, M_eff = B_step * n_q/kv.
  * Appendix B.11: prefix-attention traffic when every request re-reads the
    prefix is B * Lp * 2 * Hkv * d * 2 bytes (16-bit K and V); the contiguous
    HOT slab is read once, Lp * 2 * Hkv * d * 2 bytes; the useful work of the
    prefix contraction (Q K^T and P V) is 4 * B * Hq * Lp * d FLOPs.
"Paged KV cache" page, "Complexity and constants": KV bytes per token per
layer are 2 * kv_heads * head_dim * bytes.

Pinned by ``tests/test_oracle_costmodel.py`` against the byte, slab and FLOP
figures Appendix B.11 prints for B = 256, Lp = 8192 and a Llama-3.1-8B head,
the M_eff examples of Section 3.6, and the page's 128 KB/token for a 32-layer
Llama-3-8B.
"""
from __future__ import annotations


def m_eff(batch: int, group_size: int) -> int:
    return batch * group_size


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    return 2 * num_kv_heads * head_dim * elem_bytes


def paged_prefix_bytes(batch: int, lp: int, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    return batch * lp * kv_bytes_per_token(num_kv_heads, head_dim, elem_bytes)


def hot_prefix_bytes(lp: int, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    return lp * kv_bytes_per_token(num_kv_heads, head_dim, elem_bytes)


def prefix_flops(batch: int, num_q_heads: int, lp: int, head_dim: int) -> int:
    return 4 * batch * num_q_heads * lp * head_dim
