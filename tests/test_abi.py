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
    assert spkv.spkv_hot_write(null, null, 0, 4, null, null, 2, 1, 128, 0, null) == A.SPKV_E_INVAL
    assert spkv.spkv_hot_write(null, null, 0, 4, null, null, 8, 1, 96, 0, null) == A.SPKV_E_INVAL
    assert spkv.spkv_reshape_and_cache(null, null, null, -1, null, null, 4, 1, 64, 0, null) == A.SPKV_E_INVAL
    assert spkv.spkv_copy_blocks(null, 1, null, null, 4, 0, 1, 64, 0, null) == A.SPKV_E_INVAL
    assert spkv.spkv_merge_states(null, null, null, null, null, null, 4, 100, null) == A.SPKV_E_INVAL
    # zero-sized work is a successful no-op
    assert spkv.spkv_reshape_and_cache(null, null, null, 0, null, null, 4, 1, 64, 0, null) == A.SPKV_OK
    assert spkv.spkv_timing_enable(0) == A.SPKV_OK
