"""Seeded synthetic workloads for single-step decode attention over a HOT/COLD KV cache.

This module only draws random numbers and records configuration.  It holds
none of the method's arithmetic: no attention, no softmax, no allocator, no
slot or address computation.  Both the CPU oracle (``oracle/``) and the HIP
path (``shared_prefix_paged_amd``) consume what it returns; neither imports
the other.

Workload shapes follow the GraniKV paper's evaluation models (Llama-3.1-8B
with 8 KV heads per rank, Qwen-2.5-14B at TP=2, Qwen-2.5-32B at TP=4; its
Table 2) and its multi-prefix setting (its Section 4.4 and Appendix B.8b).
Those experiments run on ShareGPT-V3 traces with trained weights, which are not
used here: every tensor is an i.i.d. N(0, 1) draw with the same shape.

Draw order for one workload (one ``numpy.random.Generator(PCG64(seed))``):
  0. prefix lengths per group (only where a range is given),
  1. suffix lengths per request (integer uniform, both ends inclusive),
  2. per group: prefix K then prefix V, each ``[Lp, Hkv, d]``,
  3. suffix K for all requests (request-major), then suffix V,
  4. Q ``[B, Hq, d]``,
  5. the COLD free-order permutation (only when slots are shuffled).
Values are float32 draws rounded to nearest-even bfloat16 when the dtype is
bf16 (kept as raw uint16 bit patterns), or kept as float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "WorkloadConfig", "Workload", "CONFIGS", "C3_LP_SWEEP", "C3_LP_LOW",
    "bf16_bits_from_f32", "make_workload", "make_custom", "StepDraws", "step_draws",
]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``.  Inputs are finite normal draws,
    so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


@dataclass(frozen=True)
class WorkloadConfig:
    """One synthetic decode-step configuration."""
    name: str
    batch: int                      # requests per step (before forks)
    num_q_heads: int                # Hq
    num_kv_heads: int               # Hkv
    head_dim: int                   # d
    dtype: str                      # "bf16" or "f32"
    prefix_len: int                 # Lp for single-prefix configs (0 = no prefix)
    suffix_range: Tuple[int, int]   # Ls ~ U[lo, hi], inclusive
    page_size: int = 1
    shuffled: bool = True
    seed: int = 0
    num_groups: int = 1
    prefix_range: Optional[Tuple[int, int]] = None  # per-group Lp ~ U[lo, hi] when set
    steps: int = 1                  # decode steps the config describes

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def requests_per_group(self) -> int:
        return self.batch // self.num_groups


# The five configurations.  Seeds 100..104 in order.
CONFIGS = {
    "C0": WorkloadConfig("C0-tiny", 4, 4, 1, 64, "f32", 256, (1, 64), 1, True, 100),
    "C1": WorkloadConfig("C1-llama8b-lp16k", 64, 32, 8, 128, "bf16", 16384, (256, 2048), 1, True, 101),
    "C2": WorkloadConfig("C2-qwen14b-tp2-lp16k", 128, 20, 4, 128, "bf16", 16384, (128, 4096), 1, True, 102),
    "C3": WorkloadConfig("C3-qwen32b-tp4", 256, 10, 2, 128, "bf16", 16384, (128, 2048), 1, True, 103),
    "C4": WorkloadConfig("C4-multiagent-8x16", 128, 32, 8, 128, "bf16", 0, (128, 4096), 1, True, 104,
                         num_groups=8, prefix_range=(2048, 16384), steps=32),
}
C3_LP_SWEEP = (4096, 8192, 16384, 32768)
C3_LP_LOW = (0, 64, 256, 1024, 2048)


@dataclass
class Workload:
    """Drawn inputs for one step.  Arrays are uint16 bf16 bits or float32."""
    cfg: WorkloadConfig
    group_prefix_len: np.ndarray          # int64 [ng]
    group_of: np.ndarray                  # int32 [B], -1 = request has no HOT prefix
    suffix_len: np.ndarray                # int64 [B] (includes the current decode token)
    prefix_k: List[np.ndarray]            # per group [Lp_g, Hkv, d]
    prefix_v: List[np.ndarray]
    suffix_k: np.ndarray                  # [sum Ls, Hkv, d], request-major
    suffix_v: np.ndarray
    q: np.ndarray                         # [B, Hq, d]
    num_cold_pages: int
    free_order: Optional[np.ndarray]      # int32 [num_cold_pages] permutation, or None
    hot_capacity: int
    suffix_offsets: np.ndarray = field(default=None)  # int64 [B+1] into suffix_k/v

    def __post_init__(self):
        if self.suffix_offsets is None:
            self.suffix_offsets = np.concatenate([[0], np.cumsum(self.suffix_len)]).astype(np.int64)

    @property
    def batch(self) -> int:
        return int(self.suffix_len.shape[0])

    def suffix_kv(self, b: int):
        lo, hi = int(self.suffix_offsets[b]), int(self.suffix_offsets[b + 1])
        return self.suffix_k[lo:hi], self.suffix_v[lo:hi]

    def prefix_len_of(self, b: int) -> int:
        g = int(self.group_of[b])
        return 0 if g < 0 else int(self.group_prefix_len[g])

    def logical_tokens(self) -> int:
        return int(sum(self.prefix_len_of(b) + int(self.suffix_len[b]) for b in range(self.batch)))


def _draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x


def cold_pages_for(total_suffix: int, batch: int, page_size: int, extra_steps: int = 32) -> int:
    """Pool sizing rule: 1.25 x (all suffix tokens + extra_steps per request), in pages,
    plus one partially filled page per request."""
    tokens = 1.25 * (total_suffix + extra_steps * batch)
    return int(math.ceil(tokens / page_size)) + batch


def make_custom(*, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
                group_prefix_len: Sequence[int], group_of: Sequence[int], suffix_len: Sequence[int],
                page_size: int = 1, shuffled: bool = True, seed: int = 0,
                extra_steps: int = 32, name: str = "custom") -> Workload:
    """A workload with explicit lengths (edge cases, ragged shapes)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lp = np.asarray(group_prefix_len, dtype=np.int64)
    gof = np.asarray(group_of, dtype=np.int32)
    ls = np.asarray(suffix_len, dtype=np.int64)
    assert gof.shape == (batch,) and ls.shape == (batch,)
    cfg = WorkloadConfig(name, batch, num_q_heads, num_kv_heads, head_dim, dtype,
                         int(lp.max()) if lp.size else 0, (int(ls.min()), int(ls.max())) if batch else (0, 0),
                         page_size, shuffled, seed, num_groups=int(lp.size))
    return _draw_tensors(rng, cfg, lp, gof, ls, extra_steps)


def _draw_tensors(rng, cfg: WorkloadConfig, lp: np.ndarray, gof: np.ndarray, ls: np.ndarray,
                  extra_steps: int) -> Workload:
    hkv, d, dt = cfg.num_kv_heads, cfg.head_dim, cfg.dtype
    pk, pv = [], []
    for g in range(lp.size):
        pk.append(_draw(rng, (int(lp[g]), hkv, d), dt))
        pv.append(_draw(rng, (int(lp[g]), hkv, d), dt))
    total = int(ls.sum())
    sk = _draw(rng, (total, hkv, d), dt)
    sv = _draw(rng, (total, hkv, d), dt)
    q = _draw(rng, (cfg.batch, cfg.num_q_heads, d), dt)
    npages = cold_pages_for(total, cfg.batch, cfg.page_size, extra_steps)
    free_order = rng.permutation(npages).astype(np.int32) if cfg.shuffled else None
    return Workload(cfg=cfg, group_prefix_len=lp, group_of=gof, suffix_len=ls,
                    prefix_k=pk, prefix_v=pv, suffix_k=sk, suffix_v=sv, q=q,
                    num_cold_pages=npages, free_order=free_order,
                    hot_capacity=int(lp.sum()))


def make_workload(cfg: WorkloadConfig, *, prefix_len: Optional[int] = None, page_size: Optional[int] = None,
                  batch: Optional[int] = None, extra_steps: int = 32) -> Workload:
    """Draw the inputs of a named configuration.

    ``prefix_len`` overrides Lp (the C3 sweep); ``page_size`` overrides P;
    ``batch`` shrinks the batch (requests keep their order; used for bounded
    oracle samples and small parity cases).
    """
    if prefix_len is not None or page_size is not None or batch is not None:
        import dataclasses
        cfg = dataclasses.replace(
            cfg,
            prefix_len=cfg.prefix_len if prefix_len is None else prefix_len,
            page_size=cfg.page_size if page_size is None else page_size,
            batch=cfg.batch if batch is None else batch)
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    ng = cfg.num_groups
    if cfg.prefix_range is not None:
        lo, hi = cfg.prefix_range
        lp = rng.integers(lo, hi, size=ng, endpoint=True).astype(np.int64)
    else:
        lp = np.full(ng, cfg.prefix_len, dtype=np.int64)
    lo, hi = cfg.suffix_range
    ls = rng.integers(lo, hi, size=cfg.batch, endpoint=True).astype(np.int64)
    per = max(1, cfg.batch // ng)
    gof = np.minimum(np.arange(cfg.batch) // per, ng - 1).astype(np.int32)
    if lp.size == 1 and lp[0] == 0:
        gof[:] = -1
        lp = np.zeros(0, dtype=np.int64)
    return _draw_tensors(rng, cfg, lp, gof, ls, extra_steps)


@dataclass
class StepDraws:
    """Fresh per-step inputs: the new token's K/V per live request, then Q."""
    k_new: np.ndarray   # [n, Hkv, d]
    v_new: np.ndarray
    q: np.ndarray       # [n, Hq, d]


def step_draws(cfg: WorkloadConfig, step: int, n_live: int, stream: int = 0) -> StepDraws:
    """Per-step draws from their own generator, seeded by (config seed, stream, step)."""
    rng = np.random.Generator(np.random.PCG64([cfg.seed, 7919 + stream, step]))
    hkv, d, dt = cfg.num_kv_heads, cfg.head_dim, cfg.dtype
    k = _draw(rng, (n_live, hkv, d), dt)
    v = _draw(rng, (n_live, hkv, d), dt)
    q = _draw(rng, (n_live, cfg.num_q_heads, d), dt)
    return StepDraws(k, v, q)
