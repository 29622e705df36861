"""ctypes declarations of include/onetrans.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library must share with torch)

MAX_LAYERS = 16
W_BF16, W_FP8_E4M3 = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "buffer too small",
          4: "cache append capacity exceeded", 5: "HIP error"}

# the in-tree build; ONETRANS_LIB names another build of the same sources (the host-sanitizer
# build the ABI tests also run against)
LIB_PATH = os.environ.get("ONETRANS_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libonetrans.so")


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("ffn_hidden", ctypes.c_int32), ("n_ns", ctypes.c_int32), ("s_len", ctypes.c_int32),
                ("q_sched", ctypes.c_int32 * MAX_LAYERS), ("append_cap", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("ns_wdtype", ctypes.c_int32), ("n_ns_user", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "s_wqkv", "s_w1", "s_w2", "s_g_attn", "s_g_ffn", "ns_wqkv", "ns_w1", "ns_w2", "ns_scale",
        "ns_g_attn", "ns_g_ffn")]


class KVCache(ctypes.Structure):
    _fields_ = [("buf", ctypes.c_void_p), ("bytes", ctypes.c_size_t), ("n_users", ctypes.c_int32),
                ("n_appended", ctypes.c_int32), ("prefilled", ctypes.c_int32), ("layout_key", ctypes.c_uint64)]


EXPORTS = {
    # name: (restype, argtypes)
    "onetrans_check_config": (ctypes.c_int, [ctypes.POINTER(Config)]),
    "onetrans_packed_weight_bytes": (ctypes.c_size_t, [ctypes.POINTER(Config)]),
    "onetrans_pack_weights": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(LayerWeights), ctypes.c_void_p,
                                             ctypes.c_size_t, ctypes.c_void_p]),
    "onetrans_kv_cache_bytes": (ctypes.c_size_t, [ctypes.POINTER(Config), ctypes.c_int32]),
    "onetrans_kv_cache_init": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.POINTER(KVCache)]),
    "onetrans_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32]),
    "onetrans_block_forward_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Config), ctypes.c_int32,
                                                                 ctypes.c_int32]),
    "onetrans_user_prefill": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.POINTER(KVCache), ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "onetrans_kv_append": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.POINTER(KVCache), ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]),
    "onetrans_score_candidates": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_void_p, ctypes.POINTER(KVCache),
                                                 ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "onetrans_score_candidates_noalloc": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_void_p,
                                                         ctypes.POINTER(KVCache), ctypes.c_int32, ctypes.c_void_p,
                                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "onetrans_block_forward": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.c_void_p]),
    "onetrans_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "onetrans_last_error": (ctypes.c_char_p, []),
    "onetrans_kv_cache_read": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(KVCache), ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "onetrans_attention_route": (ctypes.c_char_p, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32]),
    "onetrans_kernel_timing_enable": (ctypes.c_int, [ctypes.c_uint32]),
    "onetrans_kernel_timing_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                                   ctypes.POINTER(ctypes.c_int64)]),
}

KERNEL_FAMILIES = ["s_qkv", "s_attn", "s_ffn_up", "s_ffn_down", "ns_qkv", "ns_attn", "ns_ffn_up", "ns_ffn_down",
                   "elementwise"]


def kernel_timing_enable(families) -> None:
    """Start per-launch event timing of the named kernel families (empty = off)."""
    mask = 0
    for f in families:
        mask |= 1 << KERNEL_FAMILIES.index(f)
    check(lib().onetrans_kernel_timing_enable(mask), "kernel_timing_enable")


def kernel_timing_read(family: str):
    """(total device milliseconds, launches) of one family since timing was enabled."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    check(lib().onetrans_kernel_timing_read(KERNEL_FAMILIES.index(family), ctypes.byref(ms), ctypes.byref(n)),
          "kernel_timing_read")
    return ms.value, n.value

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -m unified_transformer_recommender_onetrans_amd.build)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


class OneTransError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = lib().onetrans_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != 0:
        raise OneTransError(status, where)
