"""OneTrans block-stack forward on MI355X (gfx950): HIP kernels behind a C ABI.

The computation runs in libonetrans.so (built in-tree from csrc/ by build.py);
this package only marshals torch tensors into the C calls declared in
include/onetrans.h.
"""
from .api import KVCache, OneTrans, make_config  # noqa: F401
from ._capi import LIB_PATH, OneTransError, lib  # noqa: F401

__all__ = ["KVCache", "OneTrans", "make_config", "LIB_PATH", "OneTransError", "lib"]
