"""Drive the C ABI for a workload: tree, device pools, plan, decode.

This is the caller's side of the library (what a model's attention layer
would do), used by the tests and the benchmark.  It only marshals data:
tokens go to ``pkvt_tree_build``; each token that needs storing has its K/V
gathered from the workload's segment arrays on the host, copied to the GPU
and written into the pools by ``pkvt_kv_scatter``; attention runs in
``pkvt_attn_decode``.  PyTorch provides device memory and the stream.
"""
from __future__ import annotations

import math
from typing import List, Optional

import numpy as np

from . import binding as B


def gather_new_tokens(w, slots: np.ndarray, layer: int):
    """K/V rows (natural [n, h, d] fp16) of the tokens whose slot is >= 0,
    in build order, with their slots."""
    ks, vs, ss = [], [], []
    pos = 0
    for u in range(w.b):
        L = w.seq_len(u)
        s = slots[pos:pos + L]
        pos += L
        need = np.nonzero(s >= 0)[0]
        if need.size == 0:
            continue
        start = 0
        for si in w.seq_paths[u]:
            seg = w.segments[si]
            n = len(seg)
            sel = need[(need >= start) & (need < start + n)]
            if sel.size:
                ks.append(seg.k[layer][sel - start])
                vs.append(seg.v[layer][sel - start])
                ss.append(s[sel])
            start += n
    if not ss:
        z = np.zeros((0, w.h, w.d), np.float16)
        return z, z, np.zeros(0, np.int64)
    return np.concatenate(ks), np.concatenate(vs), np.concatenate(ss).astype(np.int64)


class DecodeSetup:
    """A built tree with per-layer K/V pools on the GPU and an uploaded plan."""

    def __init__(self, w, layers: Optional[int] = None, pool_slack: int = 0, device: str = "cuda",
                 phase1_chunks: int = 0, phase2_chunks: int = 0, min_share: int = 0,
                 pool_chunks: Optional[int] = None, unit_rows: int = 0):
        import torch
        self.torch = torch
        self.w = w
        self.layers = w.layers if layers is None else layers
        self.device = device
        total_tokens = sum(w.seq_len(u) for u in range(w.b))
        if pool_chunks is None:
            # enough for a tree with nothing shared, plus slack
            pool_chunks = sum(-(-w.seq_len(u) // w.c) for u in range(w.b)) + pool_slack
        self.pool_chunks = pool_chunks
        self.tree = B.pkvt_tree_create(w.h, w.d, w.c, pool_chunks)
        self.seq_ids, self.slots = B.pkvt_tree_build(self.tree, w.all_seq_tokens())
        assert self.slots.shape[0] == total_tokens
        pool_elems = B.pkvt_pool_bytes(w.h, w.d, w.c, pool_chunks) // 2
        self.k_pools: List = []
        self.v_pools: List = []
        stream = torch.cuda.current_stream().cuda_stream
        for layer in range(self.layers):
            kp = torch.empty(pool_elems, dtype=torch.float16, device=device)
            vp = torch.empty(pool_elems, dtype=torch.float16, device=device)
            k_new, v_new, s_new = gather_new_tokens(w, self.slots, layer)
            if s_new.size:
                kd = torch.from_numpy(np.ascontiguousarray(k_new)).to(device)
                vd = torch.from_numpy(np.ascontiguousarray(v_new)).to(device)
                sd = torch.from_numpy(s_new).to(device)
                B.pkvt_kv_scatter(self.tree, kp.data_ptr(), vp.data_ptr(), sd.data_ptr(),
                                  kd.data_ptr(), vd.data_ptr(), s_new.size, stream)
                torch.cuda.synchronize()
                del kd, vd, sd
            self.k_pools.append(kp)
            self.v_pools.append(vp)
        self.q = torch.from_numpy(np.ascontiguousarray(w.q)).to(device)
        self.out = torch.empty_like(self.q)
        self.scale = 1.0 / math.sqrt(w.d)
        self.replan(phase1_chunks, phase2_chunks, min_share, unit_rows=unit_rows)

    def replan(self, phase1_chunks: int = 0, phase2_chunks: int = 0, min_share: int = 0,
               q_order=None, unit_rows: int = 0):
        torch = self.torch
        order = self.seq_ids if q_order is None else np.asarray(q_order, np.int32)
        mb, wb = B.pkvt_plan(self.tree, order, phase1_chunks, phase2_chunks, min_share,
                             unit_rows=unit_rows)
        self.meta = torch.empty(max(mb // 4, 1), dtype=torch.int32, device=self.device)
        self.meta_bytes = mb
        self.ws = torch.empty(max(wb // 4, 1), dtype=torch.float32, device=self.device)
        self.ws_bytes = wb
        B.pkvt_plan_upload(self.tree, self.meta.data_ptr(), mb,
                           torch.cuda.current_stream().cuda_stream)
        self.info = B.pkvt_plan_info_get(self.tree)
        return self.info

    def decode(self, layer: int = 0, out=None, stream: Optional[int] = None):
        torch = self.torch
        out = self.out if out is None else out
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        B.pkvt_attn_decode(self.tree, self.meta.data_ptr(), self.q.data_ptr(),
                           self.k_pools[layer].data_ptr(), self.v_pools[layer].data_ptr(),
                           out.data_ptr(), self.ws.data_ptr() if self.ws_bytes else 0,
                           self.ws_bytes, self.scale, stream)
        return out

    def close(self):
        if self.tree:
            B.pkvt_tree_destroy(self.tree)
            self.tree = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
