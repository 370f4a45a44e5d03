"""Argument marshalling around the C ABI: numpy / torch in, ctypes out.

Nothing here computes any part of the method; each helper fills the structs
and pointers of one ``spkv_*`` call and raises on a non-zero status.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import lib, check, OutOfMemory
from . import _abi as A


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(C.POINTER(ctype))


# --------------------------------------------------------------------------- host pools

class HotPool:
    """HOT slab pool (spkv_hot_*)."""

    def __init__(self, capacity: int):
        h = C.c_void_p()
        check(lib.spkv_hot_create(int(capacity), C.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib.spkv_hot_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, lp: int) -> int:
        base = C.c_int64()
        check(lib.spkv_hot_alloc(self._h, int(lp), C.byref(base)))
        return base.value

    def incref(self, base: int):
        check(lib.spkv_hot_incref(self._h, int(base)))

    def decref(self, base: int):
        check(lib.spkv_hot_decref(self._h, int(base)))

    def evict_unreferenced(self) -> int:
        n = C.c_int32()
        check(lib.spkv_hot_evict_unreferenced(self._h, C.byref(n)))
        return n.value

    def info(self) -> A.spkv_hot_info:
        inf = A.spkv_hot_info()
        check(lib.spkv_hot_get_info(self._h, C.byref(inf)))
        return inf

    def state(self) -> dict:
        inf = self.info()
        nf, ns = inf.num_free_ranges, inf.num_slabs
        fb, fl = np.zeros(max(nf, 1), np.int64), np.zeros(max(nf, 1), np.int64)
        check(lib.spkv_hot_free_ranges(self._h, _ptr(fb, C.c_int64), _ptr(fl, C.c_int64), nf))
        sb, sl = np.zeros(max(ns, 1), np.int64), np.zeros(max(ns, 1), np.int64)
        sr, su = np.zeros(max(ns, 1), np.int32), np.zeros(max(ns, 1), np.int64)
        check(lib.spkv_hot_slabs(self._h, _ptr(sb, C.c_int64), _ptr(sl, C.c_int64), _ptr(sr, C.c_int32),
                                 _ptr(su, C.c_int64), ns))
        return {"free": [(int(fb[i]), int(fl[i])) for i in range(nf)],
                "slabs": [(int(sb[i]), int(sl[i]), int(sr[i]), int(su[i])) for i in range(ns)],
                "tick": int(inf.tick)}


class ColdPool:
    """COLD page pool (spkv_cold_*)."""

    def __init__(self, num_pages: int, page_size: int, free_order: Optional[Sequence[int]] = None):
        h = C.c_void_p()
        fo = None
        if free_order is not None:
            self._fo = np.ascontiguousarray(free_order, dtype=np.int32)
            fo = _ptr(self._fo, C.c_int32)
        check(lib.spkv_cold_create(int(num_pages), int(page_size), fo, C.byref(h)))
        self._h = h
        self.num_pages, self.page_size = int(num_pages), int(page_size)

    def close(self):
        if self._h:
            lib.spkv_cold_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seq_new(self) -> int:
        s = C.c_int32()
        check(lib.spkv_seq_new(self._h, C.byref(s)))
        return s.value

    def append_batch_raw(self, seqs: Sequence[int]):
        """Returns (status, slots[:n_done], cow pairs, n_done) without raising."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = seqs.size
        slots = np.zeros(max(n, 1), np.int32)
        cows = np.zeros(max(2 * n, 2), np.int32)
        ncow, ndone = C.c_int32(), C.c_int32()
        st = lib.spkv_cold_append_batch(self._h, _ptr(seqs, C.c_int32), n, _ptr(slots, C.c_int32),
                                        _ptr(cows, C.c_int32), C.byref(ncow), C.byref(ndone))
        pairs = [(int(cows[2 * i]), int(cows[2 * i + 1])) for i in range(ncow.value)]
        return st, slots[:ndone.value].copy(), pairs, ndone.value

    def append_batch(self, seqs: Sequence[int]):
        st, slots, pairs, n = self.append_batch_raw(seqs)
        check(st)
        return slots, pairs

    def append(self, sid: int):
        slots, pairs = self.append_batch([sid])
        return int(slots[0]), (pairs[0] if pairs else None)

    def fork(self, sid: int) -> int:
        d = C.c_int32()
        check(lib.spkv_cold_fork(self._h, int(sid), C.byref(d)))
        return d.value

    def release(self, sid: int):
        check(lib.spkv_cold_release(self._h, int(sid)))

    def block_tables(self, seqs: Sequence[int], max_blocks: int):
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = seqs.size
        tables = np.zeros((max(n, 1), max(max_blocks, 1)), np.int32)
        lens = np.zeros(max(n, 1), np.int32)
        check(lib.spkv_cold_block_tables(self._h, _ptr(seqs, C.c_int32), n, int(max_blocks),
                                         _ptr(tables, C.c_int32), _ptr(lens, C.c_int32)))
        return tables[:n, :max_blocks].copy(), lens[:n].copy()

    def info(self) -> A.spkv_cold_info:
        inf = A.spkv_cold_info()
        check(lib.spkv_cold_get_info(self._h, C.byref(inf)))
        return inf

    def seq_info(self, sid: int) -> Tuple[int, bool, int]:
        ln, live, nb = C.c_int32(), C.c_int32(), C.c_int32()
        check(lib.spkv_cold_seq_info(self._h, int(sid), C.byref(ln), C.byref(live), C.byref(nb)))
        return ln.value, bool(live.value), nb.value

    def num_free(self) -> int:
        return self.info().num_free

    def state(self) -> dict:
        inf = self.info()
        ref = np.zeros(max(inf.num_pages, 1), np.int32)
        check(lib.spkv_cold_refcounts(self._h, _ptr(ref, C.c_int32)))
        free = np.zeros(max(inf.num_free, 1), np.int32)
        check(lib.spkv_cold_free_stack(self._h, _ptr(free, C.c_int32)))
        seqs = {}
        for sid in range(inf.num_ids):
            ln, live, nb = self.seq_info(sid)
            if live:
                t, l = self.block_tables([sid], nb)
                seqs[sid] = (tuple(int(x) for x in t[0]), int(l[0]))
        return {"ref": [int(x) for x in ref[:inf.num_pages]], "free": [int(x) for x in free[:inf.num_free]],
                "seqs": seqs, "next_id": inf.num_ids}


# --------------------------------------------------------------------------- device side

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return A.SPKV_DTYPE_BF16
    if t.dtype == torch.float32:
        return A.SPKV_DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def stream_handle(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dp(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def hot_write(k_src, v_src, base: int, k_hot, v_hot, hot_capacity: int, num_kv_heads: int, head_dim: int,
              stream=None, num_layers: int = 1, layer: int = 0):
    check(lib.spkv_hot_write(_dp(k_src), _dp(v_src), int(base), int(k_src.shape[0]), _dp(k_hot), _dp(v_hot),
                             int(hot_capacity), int(num_layers), int(layer), int(num_kv_heads), int(head_dim),
                             dtype_code(k_hot), stream_handle(stream)))


def reshape_and_cache(k_new, v_new, slot_mapping, k_cold, v_cold, cold_slots: int, num_kv_heads: int,
                      head_dim: int, stream=None):
    check(lib.spkv_reshape_and_cache(_dp(k_new), _dp(v_new), _dp(slot_mapping), int(slot_mapping.numel()),
                                     _dp(k_cold), _dp(v_cold), int(cold_slots), int(num_kv_heads), int(head_dim),
                                     dtype_code(k_cold), stream_handle(stream)))


def copy_blocks(pairs, k_cold, v_cold, num_pages: int, page_size: int, num_kv_heads: int, head_dim: int,
                stream=None, num_layers: int = 1):
    n = int(pairs.numel() // 2)
    check(lib.spkv_copy_blocks(_dp(pairs) if n else None, n, _dp(k_cold), _dp(v_cold), int(num_pages),
                               int(page_size), int(num_layers), int(num_kv_heads), int(head_dim), dtype_code(k_cold),
                               stream_handle(stream)))


def block_table_append(tables, max_blocks: int, lens, rows, slots, page_size: int, stream=None):
    """Device tables/lens follow one append per listed row (spkv_block_table_append)."""
    check(lib.spkv_block_table_append(_dp(tables), int(max_blocks), _dp(lens), int(lens.numel()), _dp(rows),
                                      _dp(slots), int(rows.numel()), int(page_size), stream_handle(stream)))


def append_tokens(k_new, v_new, slots: np.ndarray, k_cold, v_cold, cold_slots: int, page_size: int,
                  num_kv_heads: int, head_dim: int, tables=None, max_blocks: int = 0, lens=None,
                  rows: Optional[np.ndarray] = None, stream=None):
    """One step's appends in one launch (spkv_append_tokens): K/V rows to their
    COLD slots and, with device tables/lens, the block-table update.  slots
    and rows are host int32 arrays (the allocator's output)."""
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n = int(slots.size)
    check(lib.spkv_append_tokens(_dp(k_new), _dp(v_new), _ptr(slots, C.c_int32),
                                 None if rows_a is None else _ptr(rows_a, C.c_int32), n, _dp(k_cold), _dp(v_cold),
                                 int(cold_slots), _dp(tables) if tables is not None else None, int(max_blocks),
                                 _dp(lens) if lens is not None else None,
                                 int(lens.numel()) if lens is not None else 0, int(page_size), int(num_kv_heads),
                                 int(head_dim), dtype_code(k_cold), stream_handle(stream)))


class KVPools:
    """Caller-owned device pools of num_layers layers; ``struct`` is the
    spkv_kv describing them for the current ``layer`` (see ``at_layer``)."""

    def __init__(self, k_hot, v_hot, hot_capacity: int, k_cold, v_cold, cold_slots: int, num_layers: int = 1,
                 layer: int = 0, row: int = 0):
        self.k_hot, self.v_hot, self.k_cold, self.v_cold = k_hot, v_hot, k_cold, v_cold
        self.hot_capacity, self.cold_slots = int(hot_capacity), int(cold_slots)
        self.num_layers, self.layer, self.row = int(num_layers), int(layer), int(row)
        self.struct = A.spkv_kv(_dp(k_hot), _dp(v_hot), self.hot_capacity, _dp(k_cold), _dp(v_cold),
                                self.cold_slots, self.num_layers, self.layer)

    def at_layer(self, layer: int) -> "KVPools":
        """The same pools, attended at another layer."""
        return KVPools(self.k_hot, self.v_hot, self.hot_capacity, self.k_cold, self.v_cold, self.cold_slots,
                       self.num_layers, layer, self.row)

    def cold_layer(self, layer: int):
        """Views of one layer's COLD K / V pool (for reshape_and_cache and append_tokens)."""
        n = self.cold_slots * self.row
        return self.k_cold[layer * n:(layer + 1) * n], self.v_cold[layer * n:(layer + 1) * n]

    @classmethod
    def allocate(cls, hot_capacity: int, cold_slots: int, num_kv_heads: int, head_dim: int, dtype, device="cuda",
                 num_layers: int = 1):
        torch = _torch()
        row = num_kv_heads * head_dim
        hot = max(hot_capacity, 1) * row * num_layers
        cold = max(cold_slots, 1) * row * num_layers
        return cls(torch.zeros(hot, dtype=dtype, device=device), torch.zeros(hot, dtype=dtype, device=device),
                   hot_capacity, torch.zeros(cold, dtype=dtype, device=device),
                   torch.zeros(cold, dtype=dtype, device=device), cold_slots, num_layers, 0, row)


class DecodeBatch:
    """Host and device arrays of one spkv_batch; keeps every buffer alive."""

    def __init__(self, q, group_of: Sequence[int], group_base: Sequence[int], group_len: Sequence[int],
                 block_tables: np.ndarray, cold_lens: Sequence[int], page_size: int, num_kv_heads: int,
                 scale: Optional[float] = None):
        torch = _torch()
        dev = q.device
        B, Hq, d = q.shape
        self.q = q.contiguous()
        self.group_of_h = np.ascontiguousarray(group_of, dtype=np.int32)
        ng = len(group_len)
        self.base_h = np.ascontiguousarray(group_base, dtype=np.int64)
        self.len_h = np.ascontiguousarray(group_len, dtype=np.int32)
        self.tables_h = np.ascontiguousarray(block_tables, dtype=np.int32)
        self.lens_h = np.ascontiguousarray(cold_lens, dtype=np.int32)
        self.max_blocks = int(self.tables_h.shape[1]) if self.tables_h.ndim == 2 else 0

        def up(a):
            return torch.from_numpy(a.copy() if a.size else np.zeros(1, a.dtype)).to(dev)

        self.group_of = up(self.group_of_h)
        self.base = up(self.base_h)
        self.len = up(self.len_h)
        self.tables = up(self.tables_h.reshape(-1))
        self.lens = up(self.lens_h)
        sc = (1.0 / float(np.sqrt(d))) if scale is None else float(scale)
        self.num_groups = ng
        self.struct = A.spkv_batch(
            int(B), int(Hq), int(num_kv_heads), int(d), dtype_code(q), sc, _dp(self.q),
            ng, _dp(self.group_of), _dp(self.base), _dp(self.len),
            self.group_of_h.ctypes.data if B else None,
            self.base_h.ctypes.data if ng else None, self.len_h.ctypes.data if ng else None,
            int(page_size), self.max_blocks, _dp(self.tables), _dp(self.lens), self.lens_h.ctypes.data)

    def workspace_size(self) -> int:
        return int(lib.spkv_workspace_size(C.byref(self.struct)))

    def plan(self, cascade: Optional[Sequence[int]] = None) -> A.spkv_plan_info:
        info = A.spkv_plan_info()
        arr = None
        if cascade is not None:
            self._casc = np.ascontiguousarray(cascade, dtype=np.int32)
            arr = _ptr(self._casc, C.c_int32)
        check(lib.spkv_plan_query(C.byref(self.struct), arr, C.byref(info)))
        return info

    def plan_parts(self, cascade: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Per-request partial-state counts (paged pass, prefix part) of the plan."""
        B = len(self.lens_h)
        flat = np.zeros(max(B, 1), dtype=np.int32)
        pre = np.zeros(max(B, 1), dtype=np.int32)
        arr = None
        if cascade is not None:
            self._casc = np.ascontiguousarray(cascade, dtype=np.int32)
            arr = _ptr(self._casc, C.c_int32)
        check(lib.spkv_plan_parts(C.byref(self.struct), arr, _ptr(flat, C.c_int32), _ptr(pre, C.c_int32)))
        return flat[:B], pre[:B]


def default_params(mode: int = A.SPKV_MODE_PER_GROUP) -> A.spkv_dispatch_params:
    p = A.spkv_dispatch_params()
    lib.spkv_dispatch_params_default(C.byref(p))
    p.mode = mode
    return p


def dispatch(batch: DecodeBatch, params: A.spkv_dispatch_params) -> np.ndarray:
    out = np.zeros(max(batch.num_groups, 1), np.int32)
    check(lib.spkv_dispatch(C.byref(batch.struct), C.byref(params), _ptr(out, C.c_int32)))
    return out[:batch.num_groups]


def _outputs(batch: DecodeBatch, out, lse):
    torch = _torch()
    B, Hq, d = batch.q.shape
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=batch.q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=batch.q.device)
    return out, lse


def workspace(batch: DecodeBatch):
    torch = _torch()
    n = batch.workspace_size()
    return torch.empty(max(n, 256), dtype=torch.uint8, device=batch.q.device)


def cascade_decode(batch: DecodeBatch, kv: KVPools, ws, out=None, lse=None, stream=None):
    out, lse = _outputs(batch, out, lse)
    check(lib.spkv_cascade_decode(C.byref(batch.struct), C.byref(kv.struct), _dp(out), _dp(lse), _dp(ws),
                                  ws.numel(), stream_handle(stream)))
    return out, lse


def dense_decode(batch: DecodeBatch, kv: KVPools, ws, out=None, lse=None, stream=None):
    out, lse = _outputs(batch, out, lse)
    check(lib.spkv_dense_decode(C.byref(batch.struct), C.byref(kv.struct), _dp(out), _dp(lse), _dp(ws),
                                ws.numel(), stream_handle(stream)))
    return out, lse


def decode_step(batch: DecodeBatch, kv: KVPools, params: A.spkv_dispatch_params, ws, out=None, lse=None,
                stream=None):
    out, lse = _outputs(batch, out, lse)
    choice = np.zeros(max(batch.num_groups, 1), np.int32)
    check(lib.spkv_decode_step(C.byref(batch.struct), C.byref(kv.struct), C.byref(params), _dp(out), _dp(lse),
                               _dp(ws), ws.numel(), stream_handle(stream), _ptr(choice, C.c_int32)))
    return out, lse, choice[:batch.num_groups]


def decode_step_append(batch: DecodeBatch, kv: KVPools, params: A.spkv_dispatch_params, ws, k_new, v_new,
                       slots: np.ndarray, out=None, lse=None, stream=None):
    """spkv_decode_step_append: the step's appends (one token per request,
    K/V rows [B, Hkv, d] on the device, host slots [B]) fused into the decode
    step.  batch.lens_h must already count the new token; the device lengths
    and block tables must not (the call advances them)."""
    out, lse = _outputs(batch, out, lse)
    choice = np.zeros(max(batch.num_groups, 1), np.int32)
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    check(lib.spkv_decode_step_append(C.byref(batch.struct), C.byref(kv.struct), C.byref(params), _dp(k_new),
                                      _dp(v_new), _ptr(slots, C.c_int32), _dp(out), _dp(lse), _dp(ws), ws.numel(),
                                      stream_handle(stream), _ptr(choice, C.c_int32)))
    return out, lse, choice[:batch.num_groups]


def decode_step_append_noalloc(batch: DecodeBatch, kv: KVPools, params: A.spkv_dispatch_params, k_new, v_new,
                               slots: np.ndarray, out=None, lse=None, stream=None):
    """spkv_decode_step_append_noalloc: decode_step_append without a workspace
    (the library's static per-device scratch holds the partial states)."""
    out, lse = _outputs(batch, out, lse)
    choice = np.zeros(max(batch.num_groups, 1), np.int32)
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    check(lib.spkv_decode_step_append_noalloc(C.byref(batch.struct), C.byref(kv.struct), C.byref(params),
                                              _dp(k_new), _dp(v_new), _ptr(slots, C.c_int32), _dp(out), _dp(lse),
                                              stream_handle(stream), _ptr(choice, C.c_int32)))
    return out, lse, choice[:batch.num_groups]


class StepGraph:
    """spkv_graph_*: the fused decode step run as a HIP graph whose kernel
    nodes take each step's arguments (see spkv_graph_decode_step_append)."""

    def __init__(self):
        h = C.c_void_p()
        check(lib.spkv_graph_create(C.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib.spkv_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def decode_step_append(self, batch: DecodeBatch, kv: KVPools, params: A.spkv_dispatch_params, ws, k_new, v_new,
                           slots: np.ndarray, out=None, lse=None, stream=None):
        """Returns (out, lse, per-group choice, instantiated)."""
        out, lse = _outputs(batch, out, lse)
        choice = np.zeros(max(batch.num_groups, 1), np.int32)
        inst = C.c_int32()
        slots = np.ascontiguousarray(slots, dtype=np.int32)
        check(lib.spkv_graph_decode_step_append(self._h, C.byref(batch.struct), C.byref(kv.struct), C.byref(params),
                                                _dp(k_new), _dp(v_new), _ptr(slots, C.c_int32), _dp(out), _dp(lse),
                                                _dp(ws), ws.numel(), stream_handle(stream),
                                                _ptr(choice, C.c_int32), C.byref(inst)))
        return out, lse, choice[:batch.num_groups], bool(inst.value)


def merge_states(o_a, lse_a, o_b, lse_b, out=None, lse=None, stream=None):
    torch = _torch()
    rows, d = o_a.shape
    out = torch.empty_like(o_a) if out is None else out
    lse = torch.empty_like(lse_a) if lse is None else lse
    check(lib.spkv_merge_states(_dp(o_a), _dp(lse_a), _dp(o_b), _dp(lse_b), _dp(out), _dp(lse), int(rows),
                                int(d), stream_handle(stream)))
    return out, lse


class KernelTimer:
    """spkv_timing_*: per-kernel-class launch durations from HIP events."""

    def __enter__(self):
        check(lib.spkv_timing_reset())
        check(lib.spkv_timing_enable(1))
        return self

    def __exit__(self, *exc):
        check(lib.spkv_timing_enable(0))

    @staticmethod
    def read(kernel: int) -> Tuple[float, int]:
        ms, n = C.c_double(), C.c_int64()
        check(lib.spkv_timing_read(int(kernel), C.byref(ms), C.byref(n)))
        return ms.value, n.value


def probe_read(buf, sink, stream=None):
    """spkv_probe_read over the bytes of a contiguous device tensor: wave w
    writes the XOR of the 32-bit words it read to sink[w] (an int32 device
    tensor of at least 4 elements, which bounds the blocks launched)."""
    torch = _torch()
    if sink.dtype != torch.int32 or sink.numel() < 4:
        raise ValueError("probe_read: sink must be int32 with at least 4 elements")
    words = int(min(sink.numel(), 2 ** 31 - 1))
    check(lib.spkv_probe_read(_dp(buf), buf.numel() * buf.element_size(), _dp(sink), words, stream_handle(stream)))


def probe_mfma(waves: int, iters: int, sink, stream=None):
    """spkv_probe_mfma: `waves` waves of `iters` rounds of 8 bf16 32x32x16
    MFMAs; one float per wave into sink (numel >= waves)."""
    torch = _torch()
    if sink.dtype != torch.float32 or sink.numel() < waves:
        raise ValueError("probe_mfma: sink must be float32 with at least `waves` elements")
    check(lib.spkv_probe_mfma(int(waves), int(iters), _dp(sink), stream_handle(stream)))
