"""fp64 CPU oracle of the OneTrans block forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .onetrans_oracle import (Layer, UserCache, append, attend, block_forward, e4m3fn_to_float, ffn,
                              forward_dense, gelu, layers_from_arrays, prefill, rmsnorm, score)

__all__ = ["Layer", "UserCache", "append", "attend", "block_forward", "e4m3fn_to_float", "ffn",
           "forward_dense", "gelu", "layers_from_arrays", "prefill", "rmsnorm", "score"]
