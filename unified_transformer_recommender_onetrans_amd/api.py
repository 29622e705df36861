"""Torch-tensor front end of the OneTrans C ABI.

Argument marshalling only: shapes and dtypes are checked, device buffers are
allocated as torch tensors, and every step of the computation runs in the HIP
library (libonetrans.so). There is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence

import torch

from . import _capi as C
from ._capi import check, lib

WEIGHT_KEYS = ("s_wqkv", "s_w1", "s_w2", "s_g_attn", "s_g_ffn", "ns_wqkv", "ns_w1", "ns_w2", "ns_scale",
               "ns_g_attn", "ns_g_ffn")


def make_config(n_layers: int, d_model: int, n_heads: int, ffn_hidden: int, n_ns: int, s_len: int,
                q_sched: Sequence[int], append_cap: int = 0, rms_eps: float = 1e-6,
                ns_wdtype: str = "bf16", n_ns_user: int = 0) -> C.Config:
    if len(q_sched) != n_layers:
        raise ValueError("q_sched needs one entry per layer")
    if n_layers > C.MAX_LAYERS:
        raise ValueError(f"at most {C.MAX_LAYERS} layers")
    cfg = C.Config()
    cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.ffn_hidden = n_layers, d_model, n_heads, ffn_hidden
    cfg.n_ns, cfg.s_len, cfg.append_cap, cfg.rms_eps = n_ns, s_len, append_cap, rms_eps
    for i, q in enumerate(q_sched):
        cfg.q_sched[i] = int(q)
    cfg.ns_wdtype = {"bf16": C.W_BF16, "e4m3": C.W_FP8_E4M3}[ns_wdtype]
    cfg.n_ns_user = n_ns_user
    return cfg


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _expect(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class KVCache:
    """A caller-owned S-side K/V cache for `n_users` users (device bytes + the C struct)."""

    def __init__(self, cfg: C.Config, n_users: int, device: torch.device):
        self.cfg = cfg
        nbytes = lib().onetrans_kv_cache_bytes(ctypes.byref(cfg), n_users)
        if nbytes == 0:
            raise ValueError("bad config or n_users")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = C.KVCache()
        check(lib().onetrans_kv_cache_init(ctypes.byref(cfg), n_users, self.buf.data_ptr(), nbytes,
                                           ctypes.byref(self.c)), "kv_cache_init")

    @property
    def n_users(self) -> int:
        return self.c.n_users

    @property
    def n_appended(self) -> int:
        return self.c.n_appended

    @property
    def prefilled(self) -> int:
        """Users [0, prefilled) hold a prefill (0 before the first one)."""
        return self.c.prefilled

    def read_layer(self, layer: int, user: int, rows: int):
        """K and V rows [0, rows) of one user and layer as bf16 [rows, d] tensors (heads concatenated)."""
        d = self.cfg.d_model
        k = torch.empty(rows, d, dtype=torch.bfloat16, device=self.buf.device)
        v = torch.empty(rows, d, dtype=torch.bfloat16, device=self.buf.device)
        check(lib().onetrans_kv_cache_read(ctypes.byref(self.cfg), ctypes.byref(self.c), layer, user, rows,
                                           k.data_ptr(), v.data_ptr(), _stream(self.buf.device)), "kv_cache_read")
        return k, v


class OneTrans:
    """The OneTrans block stack with its weights packed on one GPU."""

    def __init__(self, cfg: C.Config, layers: List[Dict[str, torch.Tensor]], device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        L, d, F, P = cfg.n_layers, cfg.d_model, cfg.ffn_hidden, cfg.n_ns
        if len(layers) != L:
            raise ValueError(f"expected {L} layer dicts")
        nsdt = torch.uint8 if cfg.ns_wdtype == C.W_FP8_E4M3 else torch.bfloat16
        shapes = {"s_wqkv": ((3 * d, d), torch.bfloat16), "s_w1": ((F, d), torch.bfloat16),
                  "s_w2": ((d, F), torch.bfloat16), "s_g_attn": ((d,), torch.float32),
                  "s_g_ffn": ((d,), torch.float32), "ns_wqkv": ((P, 3 * d, d), nsdt),
                  "ns_w1": ((P, F, d), nsdt), "ns_w2": ((P, d, F), nsdt), "ns_scale": ((P, 5), torch.float32),
                  "ns_g_attn": ((P, d), torch.float32), "ns_g_ffn": ((P, d), torch.float32)}
        arr = (C.LayerWeights * L)()
        for l, lw in enumerate(layers):
            for key in WEIGHT_KEYS:
                t = lw.get(key)
                if key == "ns_scale" and cfg.ns_wdtype == C.W_BF16:
                    setattr(arr[l], key, None)
                    continue
                _expect(t, f"layer {l} {key}", shapes[key][0], shapes[key][1], self.device)
                setattr(arr[l], key, t.data_ptr())
        nbytes = lib().onetrans_packed_weight_bytes(ctypes.byref(cfg))
        if nbytes == 0:
            check(lib().onetrans_check_config(ctypes.byref(cfg)), "config")
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        check(lib().onetrans_pack_weights(ctypes.byref(cfg), arr, self.packed.data_ptr(), nbytes,
                                          _stream(self.device)), "pack_weights")
        self._ws = torch.empty(0, dtype=torch.uint8, device=self.device)

    # -- helpers --
    def workspace(self, nbytes: int) -> torch.Tensor:
        if self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self._ws

    def new_cache(self, n_users: int) -> KVCache:
        return KVCache(self.cfg, n_users, self.device)

    @property
    def n_cand_ns(self) -> int:
        """NS rows per candidate (the positions after the user-side ones)."""
        return self.cfg.n_ns - self.cfg.n_ns_user

    def _user_ns(self, t: Optional[torch.Tensor], B: int) -> Optional[int]:
        Pu = self.cfg.n_ns_user
        if Pu == 0:
            if t is not None:
                raise ValueError("ns_user_tokens given but the config has n_ns_user = 0")
            return None
        if t is None:
            raise ValueError(f"ns_user_tokens [B, {Pu}, d] required (n_ns_user = {Pu})")
        _expect(t, "ns_user_tokens", (B, Pu, self.cfg.d_model), torch.bfloat16, self.device)
        return t.data_ptr()

    # -- the four entry points --
    def user_prefill(self, s_tokens: torch.Tensor, s_lens: torch.Tensor, cache: KVCache,
                     ns_user_tokens: Optional[torch.Tensor] = None, return_user_ns: bool = False):
        """S side (and the user-side NS rows) of B users into `cache`. Returns the S tail,
        and with return_user_ns also the user NS rows' outputs [B, n_ns_user, d]."""
        cfg = self.cfg
        B = s_tokens.shape[0]
        _expect(s_tokens, "s_tokens", (B, cfg.s_len, cfg.d_model), torch.bfloat16, self.device)
        _expect(s_lens, "s_lens", (B,), torch.int32, self.device)
        un = self._user_ns(ns_user_tokens, B)
        out = torch.empty(B, cfg.q_sched[cfg.n_layers - 1], cfg.d_model, dtype=torch.float32, device=self.device)
        un_out = (torch.empty(B, cfg.n_ns_user, cfg.d_model, dtype=torch.float32, device=self.device)
                  if return_user_ns and cfg.n_ns_user > 0 else None)
        ws = self.workspace(lib().onetrans_workspace_bytes(ctypes.byref(cfg), B, 0, 0))
        check(lib().onetrans_user_prefill(ctypes.byref(cfg), self.packed.data_ptr(), s_tokens.data_ptr(),
                                          s_lens.data_ptr(), B, un, ctypes.byref(cache.c), out.data_ptr(),
                                          _ptr(un_out), ws.data_ptr(), ws.numel(), _stream(self.device)),
              "user_prefill")
        return (out, un_out) if return_user_ns else out

    def kv_append(self, new_tokens: torch.Tensor, cache: KVCache) -> torch.Tensor:
        """m new events for each prefilled user: new_tokens [cache.prefilled, m, d]."""
        cfg = self.cfg
        B, m = cache.prefilled, new_tokens.shape[1]
        _expect(new_tokens, "new_tokens", (B, m, cfg.d_model), torch.bfloat16, self.device)
        out = torch.empty(B, m, cfg.d_model, dtype=torch.float32, device=self.device)
        ws = self.workspace(lib().onetrans_workspace_bytes(ctypes.byref(cfg), B, 0, m))
        check(lib().onetrans_kv_append(ctypes.byref(cfg), self.packed.data_ptr(), new_tokens.data_ptr(), m,
                                       ctypes.byref(cache.c), out.data_ptr(), ws.data_ptr(), ws.numel(),
                                       _stream(self.device)), "kv_append")
        return out

    def score_candidates(self, cache: KVCache, user: int, ns_tokens: torch.Tensor,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
        cfg = self.cfg
        Cn, Pc = ns_tokens.shape[0], self.n_cand_ns
        _expect(ns_tokens, "ns_tokens", (Cn, Pc, cfg.d_model), torch.bfloat16, self.device)
        if out is None:
            out = torch.empty(Cn, Pc, cfg.d_model, dtype=torch.float32, device=self.device)
        _expect(out, "ns_out", (Cn, Pc, cfg.d_model), torch.float32, self.device)
        ws = self.workspace(lib().onetrans_workspace_bytes(ctypes.byref(cfg), 0, Cn, 0))
        check(lib().onetrans_score_candidates(ctypes.byref(cfg), self.packed.data_ptr(), ctypes.byref(cache.c), user,
                                              ns_tokens.data_ptr(), Cn, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                              _stream(self.device)), "score_candidates")
        return out

    def score_candidates_noalloc(self, cache: KVCache, user: int, ns_tokens: torch.Tensor,
                                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """score_candidates through the allocation-free entry point (the library's static
        per-GPU scratch instead of a workspace; no device allocation when `out` is given)."""
        cfg = self.cfg
        Cn, Pc = ns_tokens.shape[0], self.n_cand_ns
        _expect(ns_tokens, "ns_tokens", (Cn, Pc, cfg.d_model), torch.bfloat16, self.device)
        if out is None:
            out = torch.empty(Cn, Pc, cfg.d_model, dtype=torch.float32, device=self.device)
        _expect(out, "ns_out", (Cn, Pc, cfg.d_model), torch.float32, self.device)
        check(lib().onetrans_score_candidates_noalloc(ctypes.byref(cfg), self.packed.data_ptr(), ctypes.byref(cache.c),
                                                      user, ns_tokens.data_ptr(), Cn, out.data_ptr(),
                                                      _stream(self.device)), "score_candidates_noalloc")
        return out

    def block_forward(self, s_tokens: torch.Tensor, s_lens: torch.Tensor, ns_tokens: torch.Tensor,
                      ns_user_tokens: Optional[torch.Tensor] = None):
        cfg = self.cfg
        B, Cn, Pc = ns_tokens.shape[0], ns_tokens.shape[1], self.n_cand_ns
        _expect(s_tokens, "s_tokens", (B, cfg.s_len, cfg.d_model), torch.bfloat16, self.device)
        _expect(s_lens, "s_lens", (B,), torch.int32, self.device)
        _expect(ns_tokens, "ns_tokens", (B, Cn, Pc, cfg.d_model), torch.bfloat16, self.device)
        un = self._user_ns(ns_user_tokens, B)
        s_out = torch.empty(B, cfg.q_sched[cfg.n_layers - 1], cfg.d_model, dtype=torch.float32, device=self.device)
        ns_out = torch.empty(B, Cn, Pc, cfg.d_model, dtype=torch.float32, device=self.device)
        ws = self.workspace(lib().onetrans_block_forward_workspace_bytes(ctypes.byref(cfg), B, Cn))
        check(lib().onetrans_block_forward(ctypes.byref(cfg), self.packed.data_ptr(), s_tokens.data_ptr(),
                                           s_lens.data_ptr(), B, un, ns_tokens.data_ptr(), Cn, s_out.data_ptr(),
                                           ns_out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(self.device)),
              "block_forward")
        return s_out, ns_out
