"""Python binding of libspkv.so: HOT/COLD KV cache and decode attention on MI355X.

Every function of ``include/spkv.h`` is available here under the same name
(``spkv_hot_create``, ``spkv_cascade_decode``, ...) with ctypes argument
marshalling only; ``runtime`` adds small wrappers that turn numpy arrays and
torch tensors into those arguments.  All computation happens in the native
library: importing this package fails if ``libspkv.so`` is missing.
"""
from __future__ import annotations

import ctypes as _C
import os as _os

from . import _abi
from ._abi import *  # noqa: F401,F403  (structs and constants)

# PyTorch ships its own HIP runtime under the same soname as ROCm's.  Loading
# torch first makes libspkv.so bind to that runtime, so device memory, streams
# and our launches live in one HIP runtime per process.
try:
    import torch as _torch  # noqa: F401
except ImportError:  # host-only use (allocators) works without torch
    _torch = None

_LIB_PATH = _os.path.join(_os.path.dirname(_os.path.abspath(__file__)), "libspkv.so")
if not _os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run `python shared_prefix_paged_amd/build.py` "
                      "(or __graft_entry__.build()) first")
lib = _C.CDLL(_LIB_PATH)
_abi.declare(lib)
LIB_PATH = _LIB_PATH

for _name in _abi.SIGNATURES:
    globals()[_name] = getattr(lib, _name)


class SpkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"spkv status {status}: {msg}")
        self.status = status


class InvalidArgument(SpkvError):
    pass


class OutOfMemory(SpkvError):
    pass


class StateError(SpkvError):
    pass


class HipError(SpkvError):
    pass


_ERRORS = {_abi.SPKV_E_INVAL: InvalidArgument, _abi.SPKV_E_NOMEM: OutOfMemory,
           _abi.SPKV_E_STATE: StateError, _abi.SPKV_E_HIP: HipError}


def check(status: int) -> None:
    """Raise the matching SpkvError for a non-zero status."""
    if status != _abi.SPKV_OK:
        msg = lib.spkv_last_error().decode(errors="replace")
        raise _ERRORS.get(status, SpkvError)(status, msg)


def version() -> str:
    return lib.spkv_version().decode()
