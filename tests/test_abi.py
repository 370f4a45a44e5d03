"""The C-ABI library loads on a machine without a GPU, exports every symbol the
header declares, and reports errors by status code (CPU only)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from conftest import ROOT
import shared_prefix_paged_amd as spkv
from shared_prefix_paged_amd import _abi as A
from shared_prefix_paged_amd.runtime import ColdPool, HotPool


def header_functions():
    text = open(os.path.join(ROOT, "include", "spkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spkv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 35
    lib = C.CDLL(spkv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} missing from libspkv.so"
    assert sorted(A.SIGNATURES) == names, "binding and header disagree"


def test_binding_names_match_header():
    for n in header_functions():
        assert callable(getattr(spkv, n))


def test_version_and_error_text():
    assert "gfx950" in spkv.version()
    st = spkv.spkv_hot_create(-5, C.byref(C.c_void_p()))
    assert st == A.SPKV_E_INVAL
    assert "hot_create" in spkv.spkv_last_error().decode()


def test_status_codes():
    hot = HotPool(8)
    with pytest.raises(spkv.InvalidArgument):
        hot.alloc(0)
    with pytest.raises(spkv.OutOfMemory):
        hot.alloc(9)
    with pytest.raises(spkv.StateError):
        hot.decref(3)
    b = hot.alloc(3)
    hot.decref(b)
    with pytest.raises(spkv.StateError):
        hot.decref(b)
    cold = ColdPool(2, 1)
    s = cold.seq_new()
    cold.append(s)
    cold.release(s)
    with pytest.raises(spkv.StateError):
        cold.release(s)
    with pytest.raises(spkv.StateError):
        cold.append(s)
    with pytest.raises(spkv.InvalidArgument):
        ColdPool(3, 1, free_order=[0, 1, 1])
    with pytest.raises(spkv.InvalidArgument):
        ColdPool(3, 0)


def test_append_batch_reports_partial_progress():
    cold = ColdPool(3, 1)
    a, b = cold.seq_new(), cold.seq_new()
    st, slots, pairs, n = cold.append_batch_raw([a, b, a, b, a])
    assert st == A.SPKV_E_NOMEM and n == 3 and list(slots) == [0, 1, 2]
    st, slots, pairs, n = cold.append_batch_raw([99, a])
    assert st == A.SPKV_E_STATE and n == 0


def test_block_tables_padding_and_bounds():
    cold = ColdPool(8, 2)
    a = cold.seq_new()
    for _ in range(5):
        cold.append(a)
    t, l = cold.block_tables([a], 4)
    assert list(t[0]) == [0, 1, 2, -1] and list(l) == [5]
    with pytest.raises(spkv.InvalidArgument):
        cold.block_tables([a], 2)


def test_device_ops_validate_before_touching_the_gpu():
    # Shape and range checks fail before any HIP call is made.
    null = None
    assert spkv.spkv_hot_write(null, null, 0, 4, null, null, 2, 1, 0, 1, 128, 0, null) == A.SPKV_E_INVAL
    assert spkv.spkv_hot_write(null, null, 0, 4, null, null, 8, 1, 0, 1, 96, 0, null) == A.SPKV_E_INVAL
    assert spkv.spkv_hot_write(null, null, 0, 4, null, null, 8, 2, 2, 1, 128, 0, null) == A.SPKV_E_INVAL  # layer 2 of 2
    assert spkv.spkv_reshape_and_cache(null, null, null, -1, null, null, 4, 1, 64, 0, null) == A.SPKV_E_INVAL
    assert spkv.spkv_copy_blocks(null, 1, null, null, 4, 0, 1, 1, 64, 0, null) == A.SPKV_E_INVAL
    assert spkv.spkv_copy_blocks(null, 1, null, null, 4, 1, 0, 1, 64, 0, null) == A.SPKV_E_INVAL  # no layers
    assert spkv.spkv_merge_states(null, null, null, null, null, null, 4, 100, null) == A.SPKV_E_INVAL
    # zero-sized work is a successful no-op
    assert spkv.spkv_reshape_and_cache(null, null, null, 0, null, null, 4, 1, 64, 0, null) == A.SPKV_OK
    assert spkv.spkv_timing_enable(0) == A.SPKV_OK


def test_append_tokens_rejects_bad_slots_and_rows_on_the_host():
    # [PKV] How it works, step 1: a token is written at its slot; a slot outside
    # the pool (or a block-table row outside the batch) is an error reported
    # before anything is launched, not a silently skipped write.
    import ctypes as C
    import numpy as np
    fake = C.c_void_p(16)                      # never dereferenced: the checks come first
    slots = np.array([0, 7, 8], np.int32)      # 8 is outside an 8-slot pool
    rows = np.array([0, 1, 2], np.int32)
    sp = slots.ctypes.data_as(C.POINTER(C.c_int32))
    rp = rows.ctypes.data_as(C.POINTER(C.c_int32))
    st = spkv.spkv_append_tokens(fake, fake, sp, rp, 3, fake, fake, 8, None, 0, None, 0, 1, 1, 64, 0, None)
    assert st == A.SPKV_E_INVAL and "outside the COLD pool" in spkv.lib.spkv_last_error().decode()
    slots[2] = -1
    assert spkv.spkv_append_tokens(fake, fake, sp, rp, 3, fake, fake, 8, None, 0, None, 0, 1, 1, 64, 0,
                                   None) == A.SPKV_E_INVAL
    slots[2] = 3
    rows[1] = 5                                # only 3 rows in the tables
    st = spkv.spkv_append_tokens(fake, fake, sp, rp, 3, fake, fake, 8, fake, 4, fake, 3, 1, 1, 64, 0, None)
    assert st == A.SPKV_E_INVAL and "row" in spkv.lib.spkv_last_error().decode()


def test_group_membership_is_group_of_alone():
    # [GKV] Section 3.4: a request records which prefix (HOT slab) it shares.
    # The batch descriptor carries only group_of and the per-group slab arrays;
    # the library forms member lists itself, so there is no second list that
    # could disagree with group_of.
    names = [f[0] for f in A.spkv_batch._fields_]
    assert "group_of" in names and not any("indptr" in n or "member" in n for n in names)
    import numpy as np
    import torch
    from shared_prefix_paged_amd import runtime as R
    q = torch.zeros((3, 8, 64), dtype=torch.bfloat16)
    tables = np.zeros((3, 1), np.int32)
    for bad in ([0, 2, -1], [0, -2, 1]):       # group 2 does not exist; -2 is not "no group"
        batch = R.DecodeBatch(q, bad, [0, 10], [10, 5], tables, [1, 1, 1], 1, 2)
        with pytest.raises(spkv.InvalidArgument):
            batch.plan()
    # at most 512 groups per step (the per-group cascade mask's size): 513 is refused
    many = R.DecodeBatch(q, [0, 1, 512], list(range(513)), [1] * 513, tables, [1, 1, 1], 1, 2)
    with pytest.raises(spkv.InvalidArgument):
        many.plan()
    ok = R.DecodeBatch(q, [0, 1, 511], list(range(512)), [1] * 512, tables, [1, 1, 1], 1, 2)
    ok.plan()
    # members counted from group_of: two groups of 2 and 1 requests, cascade planned for both
    batch = R.DecodeBatch(q, [1, 0, 1], [0, 300], [300, 300], tables, [1, 1, 1], 1, 2)
    fp, pp = batch.plan_parts()
    assert list(pp > 0) == [True, True, True]


def test_noalloc_rejects_plans_beyond_its_scratch_before_launching():
    # The entry point without a workspace refuses, on the host, a step whose
    # plan needs more than its static scratch (2048 requests x 32 heads).
    import torch
    from shared_prefix_paged_amd import runtime as R
    B = 2048
    q = torch.zeros((B, 32, 128), dtype=torch.bfloat16)
    batch = R.DecodeBatch(q, [0] * B, [0], [4096], np.zeros((B, 64), np.int32), [60] * B, 1, 8)
    assert batch.plan().workspace_bytes > A.SPKV_NOALLOC_SCRATCH_BYTES
    fake = C.c_void_p(16)
    kv = A.spkv_kv(16, 16, 4096, 16, 16, 1 << 20, 1, 0)
    slots = np.arange(B, dtype=np.int32)
    st = spkv.spkv_decode_step_append_noalloc(C.byref(batch.struct), C.byref(kv),
                                              C.byref(R.default_params()), fake, fake,
                                              slots.ctypes.data_as(C.POINTER(C.c_int32)), fake, fake, None, None)
    assert st == A.SPKV_E_INVAL and "static" in spkv.lib.spkv_last_error().decode()


def test_empty_batch_is_a_no_op_without_touching_the_device():
    # B = 0: every decode entry point validates and returns SPKV_OK before any
    # device call (this runs on a machine without a GPU).
    b = A.spkv_batch()
    b.batch, b.num_q_heads, b.num_kv_heads, b.head_dim = 0, 8, 2, 128
    b.dtype, b.scale, b.page_size, b.max_blocks = A.SPKV_DTYPE_BF16, 0.088, 1, 0
    kv = A.spkv_kv()
    kv.num_layers, kv.layer = 1, 0
    from shared_prefix_paged_amd import runtime as R
    params = R.default_params()
    assert spkv.spkv_cascade_decode(C.byref(b), C.byref(kv), None, None, None, 0, None) == A.SPKV_OK
    assert spkv.spkv_dense_decode(C.byref(b), C.byref(kv), None, None, None, 0, None) == A.SPKV_OK
    assert spkv.spkv_decode_step(C.byref(b), C.byref(kv), C.byref(params), None, None, None, 0, None, None) == A.SPKV_OK
    assert spkv.spkv_workspace_size(C.byref(b)) > 0
    info = A.spkv_plan_info()
    assert spkv.spkv_plan_query(C.byref(b), None, C.byref(info)) == A.SPKV_OK
    assert info.single_launch == 0 and info.flat_items == 0 and info.prefix_items == 0
