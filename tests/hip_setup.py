"""Loads a drawn workload onto the GPU through the C ABI (native allocators,
hot_write, reshape_and_cache, copy_blocks), in the same operation order as the
oracle driver, so slots, tables and pools can be compared bit for bit."""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from shared_prefix_paged_amd import runtime as R


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def pool_bytes(t: torch.Tensor) -> np.ndarray:
    """Raw contents of a device pool as uint16 (bf16) or float32 numpy array."""
    h = t.detach().cpu()
    if h.dtype == torch.bfloat16:
        return h.view(torch.int16).numpy().view(np.uint16)
    return h.numpy()


@dataclass
class GpuStep:
    hot: R.HotPool
    cold: R.ColdPool
    bases: List[int]
    seqs: List[int]
    setup_slots: np.ndarray
    step_slots: np.ndarray
    step_cows: list
    tables: np.ndarray
    lens: np.ndarray
    pools: R.KVPools
    batch: R.DecodeBatch
    page_size: int


def members_per_group(wl) -> np.ndarray:
    return np.bincount(wl.group_of[wl.group_of >= 0], minlength=len(wl.group_prefix_len))


def setup_single_step(wl, page_size: Optional[int] = None, free_order=None, device="cuda",
                      max_blocks: Optional[int] = None, num_layers: int = 1) -> GpuStep:
    """num_layers > 1: pools of that many layers (one HOT and one COLD
    allocation), every layer holding the workload's K/V; attention reads the
    layer set in the returned pools (pools.at_layer(l) for another)."""
    cfg = wl.cfg
    P = cfg.page_size if page_size is None else page_size
    hkv, d = cfg.num_kv_heads, cfg.head_dim
    hot = R.HotPool(wl.hot_capacity)
    counts = members_per_group(wl)
    bases = []
    for g, lp in enumerate(wl.group_prefix_len):
        base = hot.alloc(int(lp))
        for _ in range(int(counts[g]) - 1):
            hot.incref(base)
        bases.append(base)
    fo = wl.free_order if free_order is None else free_order
    cold = R.ColdPool(wl.num_cold_pages, P, fo)
    B = wl.batch
    seqs = [cold.seq_new() for _ in range(B)]
    setup_ids = [seqs[b] for b in range(B) for _ in range(int(wl.suffix_len[b]) - 1)]
    setup_slots, _ = cold.append_batch(setup_ids) if setup_ids else (np.zeros(0, np.int32), [])
    step_slots, step_cows = cold.append_batch(seqs) if B else (np.zeros(0, np.int32), [])

    pools = R.KVPools.allocate(wl.hot_capacity, wl.num_cold_pages * P, hkv, d, torch_dtype(cfg.dtype), device,
                               num_layers=num_layers)
    for layer in range(num_layers):
        for g, base in enumerate(bases):
            R.hot_write(to_device(wl.prefix_k[g], cfg.dtype, device), to_device(wl.prefix_v[g], cfg.dtype, device),
                        base, pools.k_hot, pools.v_hot, wl.hot_capacity, hkv, d, num_layers=num_layers, layer=layer)
    off = wl.suffix_offsets
    if len(setup_slots):
        rows = np.concatenate([np.arange(off[b], off[b + 1] - 1) for b in range(B)])
        ks, vs = to_device(wl.suffix_k[rows], cfg.dtype, device), to_device(wl.suffix_v[rows], cfg.dtype, device)
        sl = torch.from_numpy(setup_slots).to(device)
        for layer in range(num_layers):
            kc, vc = pools.cold_layer(layer)
            R.reshape_and_cache(ks, vs, sl, kc, vc, pools.cold_slots, hkv, d)
    if step_cows:
        R.copy_blocks(torch.tensor(step_cows, dtype=torch.int32, device=device), pools.k_cold, pools.v_cold,
                      wl.num_cold_pages, P, hkv, d, num_layers=num_layers)
    if B:
        last = off[1:] - 1
        ks, vs = to_device(wl.suffix_k[last], cfg.dtype, device), to_device(wl.suffix_v[last], cfg.dtype, device)
        sl = torch.from_numpy(np.asarray(step_slots, np.int32)).to(device)
        for layer in range(num_layers):
            kc, vc = pools.cold_layer(layer)
            R.reshape_and_cache(ks, vs, sl, kc, vc, pools.cold_slots, hkv, d)
    lens_now = [cold.seq_info(s)[0] for s in seqs]
    need = max([(l + P - 1) // P for l in lens_now] + [1])
    mb = need if max_blocks is None else max(max_blocks, need)
    tables, lens = cold.block_tables(seqs, mb) if B else (np.zeros((0, mb), np.int32), np.zeros(0, np.int32))
    q = to_device(wl.q, cfg.dtype, device)
    batch = R.DecodeBatch(q, wl.group_of, bases, wl.group_prefix_len, tables, lens, P, hkv)
    return GpuStep(hot, cold, bases, seqs, np.asarray(setup_slots), np.asarray(step_slots), step_cows, tables,
                   lens, pools, batch, P)


def errors(out: torch.Tensor, lse: torch.Tensor, ref_o: np.ndarray, ref_l: np.ndarray, rows=None):
    o = out.detach().cpu().double().numpy()
    l = lse.detach().cpu().double().numpy()
    if rows is not None:
        o, l, ref_o, ref_l = o[rows], l[rows], ref_o[rows], ref_l[rows]
    max_abs = float(np.max(np.abs(o - ref_o))) if o.size else 0.0
    lse_abs = float(np.max(np.abs(l - ref_l))) if l.size else 0.0
    rel = float(np.linalg.norm(o - ref_o) / max(np.linalg.norm(ref_o), 1e-30)) if o.size else 0.0
    return max_abs, lse_abs, rel
