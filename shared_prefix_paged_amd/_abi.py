"""ctypes declarations of every function and struct in include/spkv.h."""
from __future__ import annotations

import ctypes as C

c_i32, c_i64, c_f32, c_f64, c_vp, c_sz = C.c_int32, C.c_int64, C.c_float, C.c_double, C.c_void_p, C.c_size_t
P_i32, P_i64, P_f32, P_f64 = C.POINTER(c_i32), C.POINTER(c_i64), C.POINTER(c_f32), C.POINTER(c_f64)

SPKV_OK, SPKV_E_INVAL, SPKV_E_NOMEM, SPKV_E_STATE, SPKV_E_HIP = 0, -1, -2, -3, -4
SPKV_DTYPE_BF16, SPKV_DTYPE_F32 = 0, 1
SPKV_MODE_PER_GROUP, SPKV_MODE_BATCH_GLOBAL, SPKV_MODE_FORCE_CASCADE, SPKV_MODE_FORCE_DENSE = 0, 1, 2, 3
SPKV_KERNEL_PREFIX, SPKV_KERNEL_FLAT, SPKV_KERNEL_MERGE, SPKV_KERNEL_CACHE = 0, 1, 2, 3
SPKV_KERNEL_PAGED_PREFIX, SPKV_NUM_KERNELS = 4, 5
SPKV_NOALLOC_SCRATCH_BYTES = 32 << 20


class spkv_hot_info(C.Structure):
    _fields_ = [("capacity", c_i64), ("free_tokens", c_i64), ("num_free_ranges", c_i32),
                ("num_slabs", c_i32), ("tick", c_i64)]


class spkv_cold_info(C.Structure):
    _fields_ = [("num_pages", c_i32), ("page_size", c_i32), ("num_free", c_i32),
                ("num_ids", c_i32), ("num_live", c_i32)]


class spkv_batch(C.Structure):
    _fields_ = [("batch", c_i32), ("num_q_heads", c_i32), ("num_kv_heads", c_i32), ("head_dim", c_i32),
                ("dtype", c_i32), ("scale", c_f32), ("q", c_vp),
                ("num_groups", c_i32), ("group_of", c_vp), ("hot_base", c_vp), ("hot_len", c_vp),
                ("host_group_of", c_vp), ("host_hot_base", c_vp), ("host_hot_len", c_vp),
                ("page_size", c_i32), ("max_blocks", c_i32), ("block_tables", c_vp), ("cold_lens", c_vp),
                ("host_cold_lens", c_vp)]


class spkv_kv(C.Structure):
    _fields_ = [("k_hot", c_vp), ("v_hot", c_vp), ("hot_capacity", c_i64),
                ("k_cold", c_vp), ("v_cold", c_vp), ("cold_slots", c_i64),
                ("num_layers", c_i32), ("layer", c_i32)]


class spkv_dispatch_params(C.Structure):
    _fields_ = [("mode", c_i32), ("min_group_requests", c_i32), ("fixed_cost_us", c_f64),
                ("flat_gbps", c_f64), ("prefix_gbps", c_f64), ("prefix_tflops", c_f64), ("row_cost_ns", c_f64),
                ("single_launch", c_i32)]


class spkv_plan_info(C.Structure):
    _fields_ = [("flat_chunk", c_i32), ("flat_splits", c_i32), ("prefix_chunk", c_i32), ("prefix_splits", c_i32),
                ("prefix_waves", c_i32), ("prefix_mtiles", c_i32), ("flat_items", c_i64),
                ("prefix_items", c_i64), ("workspace_bytes", c_i64), ("flat_split_cap", c_i32),
                ("flat_head_tokens", c_i32), ("prefix_split_cap", c_i32), ("prefix_granule", c_i32),
                ("prefix_key_halves", c_i32), ("single_launch", c_i32), ("co_resident", c_i32),
                ("co_prefix_stages", c_i32)]


P_batch, P_kv, P_params = C.POINTER(spkv_batch), C.POINTER(spkv_kv), C.POINTER(spkv_dispatch_params)

# name -> (restype, argtypes); the order follows include/spkv.h.
SIGNATURES = {
    "spkv_last_error": (C.c_char_p, []),
    "spkv_version": (C.c_char_p, []),
    "spkv_hot_create": (c_i32, [c_i64, C.POINTER(c_vp)]),
    "spkv_hot_destroy": (None, [c_vp]),
    "spkv_hot_alloc": (c_i32, [c_vp, c_i64, P_i64]),
    "spkv_hot_incref": (c_i32, [c_vp, c_i64]),
    "spkv_hot_decref": (c_i32, [c_vp, c_i64]),
    "spkv_hot_evict_unreferenced": (c_i32, [c_vp, P_i32]),
    "spkv_hot_get_info": (c_i32, [c_vp, C.POINTER(spkv_hot_info)]),
    "spkv_hot_free_ranges": (c_i32, [c_vp, P_i64, P_i64, c_i32]),
    "spkv_hot_slabs": (c_i32, [c_vp, P_i64, P_i64, P_i32, P_i64, c_i32]),
    "spkv_cold_create": (c_i32, [c_i32, c_i32, P_i32, C.POINTER(c_vp)]),
    "spkv_cold_destroy": (None, [c_vp]),
    "spkv_seq_new": (c_i32, [c_vp, P_i32]),
    "spkv_cold_append_batch": (c_i32, [c_vp, P_i32, c_i32, P_i32, P_i32, P_i32, P_i32]),
    "spkv_cold_fork": (c_i32, [c_vp, c_i32, P_i32]),
    "spkv_cold_release": (c_i32, [c_vp, c_i32]),
    "spkv_cold_block_tables": (c_i32, [c_vp, P_i32, c_i32, c_i32, P_i32, P_i32]),
    "spkv_cold_get_info": (c_i32, [c_vp, C.POINTER(spkv_cold_info)]),
    "spkv_cold_refcounts": (c_i32, [c_vp, P_i32]),
    "spkv_cold_free_stack": (c_i32, [c_vp, P_i32]),
    "spkv_cold_seq_info": (c_i32, [c_vp, c_i32, P_i32, P_i32, P_i32]),
    "spkv_hot_write": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_i64, c_i32, c_i32, c_i32, c_i32, c_i32,
                               c_vp]),
    "spkv_reshape_and_cache": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i64, c_i32, c_i32, c_i32, c_vp]),
    "spkv_copy_blocks": (c_i32, [c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "spkv_block_table_append": (c_i32, [c_vp, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_vp]),
    "spkv_append_tokens": (c_i32, [c_vp, c_vp, P_i32, P_i32, c_i32, c_vp, c_vp, c_i64, c_vp, c_i32, c_vp, c_i32,
                                   c_i32, c_i32, c_i32, c_i32, c_vp]),
    "spkv_workspace_size": (c_sz, [P_batch]),
    "spkv_cascade_decode": (c_i32, [P_batch, P_kv, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "spkv_dense_decode": (c_i32, [P_batch, P_kv, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "spkv_merge_states": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_vp]),
    "spkv_dispatch_params_default": (None, [P_params]),
    "spkv_dispatch": (c_i32, [P_batch, P_params, P_i32]),
    "spkv_decode_step": (c_i32, [P_batch, P_kv, P_params, c_vp, c_vp, c_vp, c_sz, c_vp, P_i32]),
    "spkv_decode_step_append": (c_i32, [P_batch, P_kv, P_params, c_vp, c_vp, P_i32, c_vp, c_vp, c_vp, c_sz, c_vp,
                                        P_i32]),
    "spkv_decode_step_append_noalloc": (c_i32, [P_batch, P_kv, P_params, c_vp, c_vp, P_i32, c_vp, c_vp, c_vp,
                                                P_i32]),
    "spkv_graph_create": (c_i32, [C.POINTER(c_vp)]),
    "spkv_graph_destroy": (None, [c_vp]),
    "spkv_graph_decode_step_append": (c_i32, [c_vp, P_batch, P_kv, P_params, c_vp, c_vp, P_i32, c_vp, c_vp, c_vp,
                                              c_sz, c_vp, P_i32, P_i32]),
    "spkv_plan_query": (c_i32, [P_batch, P_i32, C.POINTER(spkv_plan_info)]),
    "spkv_plan_parts": (c_i32, [P_batch, P_i32, P_i32, P_i32]),
    "spkv_timing_enable": (c_i32, [c_i32]),
    "spkv_timing_read": (c_i32, [c_i32, P_f64, P_i64]),
    "spkv_timing_reset": (c_i32, []),
    "spkv_device_cus": (c_i32, [P_i32]),
    "spkv_probe_read": (c_i32, [c_vp, c_sz, c_vp, c_i32, c_vp]),
    "spkv_probe_mfma": (c_i32, [c_i32, c_i32, c_vp, c_vp]),
}


def declare(lib) -> None:
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
