"""One ETA decode step over a resident KV cache, as a sequence of C-ABI calls.

``DecodeStep`` owns the per-step device buffers (tau, admitted lists, outputs,
workspace) for one cache of B rows, H query heads and H_kv key/value heads
(H_kv = H: multi-head attention) and enqueues the library calls of a step on
the current stream with no host synchronisation:
eta_predict_tau + eta_screen [-> eta_admit_union for grouped heads], or in one
launch eta_predict_screen (eta_predict_screen_union for grouped heads)
-> eta_decode_attn
(= eta_decode_attn_partial followed by eta_decode_attn_combine).

With ``layout`` (a ``_lib.KVLayout``) the rows hold their own lengths and/or the
K/V bytes live in a page pool; the step reads the layout's tensors at run time,
so a captured graph follows in-place updates of the lengths and page table.
"""
from __future__ import annotations

import torch

from . import _lib


class DecodeStep:
    def __init__(self, B, H, d, T_cap, kv_dtype=torch.bfloat16, params=None, device="cuda",
                 with_bounds=False, H_kv=None, layout=None):
        self.B, self.H, self.d, self.T_cap = B, H, d, T_cap
        self.layout = layout
        self.H_kv = H if H_kv is None else H_kv
        self.G = H // self.H_kv
        self.kv_dtype = kv_dtype
        self.params = params if params is not None else _lib.default_params()
        n = _lib.nblk_cap(T_cap)
        self.tau = torch.empty((B, H), dtype=torch.float32, device=device)
        self.adm_idx = torch.empty((B, H, n), dtype=torch.int32, device=device)
        self.adm_cnt = torch.empty((B, H), dtype=torch.int32, device=device)
        if self.G > 1:
            self.uni_idx = torch.empty((B, self.H_kv, n), dtype=torch.int32, device=device)
            self.uni_cnt = torch.empty((B, self.H_kv), dtype=torch.int32, device=device)
        else:  # multi-head: the attention reads the screen's lists directly
            self.uni_idx, self.uni_cnt = self.adm_idx, self.adm_cnt
        self.out = torch.empty((B, H, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=device)
        self.bounds = (torch.empty((B, H, n), dtype=torch.float32, device=device)
                       if with_bounds else None)
        self._hkv_arg = 0 if self.G == 1 else self.H_kv
        self.ws = _lib.alloc_workspace(B, H, d, T_cap, self.params, kv_dtype, device,
                                       self._hkv_arg)

    def predict(self, q, W, bias, stream=None):
        _lib.eta_predict_tau(q, W, bias, self.tau, stream)

    def predict_screen(self, q, W, bias, meta, T, stream=None):
        if self.G > 1:  # the union comes out of the same launch
            _lib.eta_predict_screen_union(q, W, bias, meta, T, self.T_cap, self.params, self.tau,
                                          self.adm_idx, self.adm_cnt, self.uni_idx, self.uni_cnt,
                                          self.bounds, self.kv_dtype, stream, self.layout)
            return
        _lib.eta_predict_screen(q, W, bias, meta, T, self.T_cap, self.params, self.tau,
                                self.adm_idx, self.adm_cnt, self.bounds, self.kv_dtype, stream,
                                self._hkv_arg, self.layout)

    def screen(self, q, meta, T, stream=None):
        _lib.eta_screen(q, self.tau, meta, T, self.T_cap, self.params, self.adm_idx,
                        self.adm_cnt, self.bounds, self.kv_dtype, stream, self._hkv_arg,
                        self.layout)
        self.union(T, stream)

    def union(self, T, stream=None):
        if self.G > 1:
            _lib.eta_admit_union(self.adm_idx, self.adm_cnt, self.uni_idx, self.uni_cnt, T,
                                 self.T_cap, self.d, self.kv_dtype, stream)

    def attend(self, q, K, V, T, stream=None):
        _lib.eta_decode_attn(q, K, V, T, self.tau, self.uni_idx, self.uni_cnt, self.params,
                             self.out, self.lse, self.ws, stream, self.layout)

    def attend_partial(self, q, K, V, T, stream=None):
        _lib.eta_decode_attn_partial(q, K, V, T, self.tau, self.uni_idx, self.uni_cnt,
                                     self.params, self.out, self.lse, self.ws, stream,
                                     self.layout)

    def attend_combine(self, K, T, stream=None):
        _lib.eta_decode_attn_combine(K, T, self.uni_cnt, self.params, self.out, self.lse,
                                     self.ws, stream, self.layout)

    def capture(self, q, K, V, T, meta, W, bias, fused=True):
        """Record one step into a HIP graph (torch.cuda.CUDAGraph) and return it; each
        replay re-runs the step on the same buffers. The library makes no allocation
        and no memset, so the captured step holds kernel nodes only."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm the launch path outside the capture
            self(q, K, V, T, meta, W, bias, fused=fused)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self(q, K, V, T, meta, W, bias, fused=fused)
        return graph

    def __call__(self, q, K, V, T, meta, W, bias, stream=None, fused=False):
        """One step; fused=True evaluates tau inside the screen launch."""
        if fused:
            self.predict_screen(q, W, bias, meta, T, stream)
        else:
            self.predict(q, W, bias, stream)
            self.screen(q, meta, T, stream)
        self.attend(q, K, V, T, stream)
        return self.out
