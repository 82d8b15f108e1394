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
                 pool_chunks: Optional[int] = None, unit_rows: int = 0,
                 device_random_seed: Optional[int] = None, match: str = "chunks",
                 build_groups: int = 1, extra_layers_seed: Optional[int] = None):
        """``device_random_seed``: instead of the workload's K/V (which may
        then be absent), fill the pools and Q with N(0,1) fp16 drawn on the
        device (for timing sweeps that need no oracle).
        ``extra_layers_seed``: ``layers`` may exceed the workload's own layer
        count; the pools of the layers it lacks are drawn N(0,1) on the
        device with this seed (Q and the workload's layers stay as given, so
        those layers can still be checked against the oracle).  ``match``: the
        tree's prefix matching ("chunks" or "tokens").  ``build_groups``:
        insert the sequences in that many successive pkvt_tree_build calls
        (in order); under token matching a later call may split nodes of an
        earlier one, whose K/V then move (pkvt_kv_move) before the new
        tokens are written."""
        import torch
        self.torch = torch
        self.w = w
        self.layers = w.layers if layers is None else layers
        self.device = device
        total_tokens = sum(w.seq_len(u) for u in range(w.b))
        if pool_chunks is None:
            # enough for a tree with nothing shared (and, under token matching,
            # one split per arrival), plus slack
            pool_chunks = sum(-(-w.seq_len(u) // w.c) for u in range(w.b)) + pool_slack
            if match == "tokens":
                pool_chunks += w.b
        self.pool_chunks = pool_chunks
        self.tree = B.pkvt_tree_create(w.h, w.d, w.c, pool_chunks, match=match)
        prompts = w.all_seq_tokens()
        bounds = np.linspace(0, w.b, max(1, build_groups) + 1).astype(int)
        ids_parts, builds = [], []           # per call: (full-length slots, move src, move dst)
        tok_at = np.cumsum([0] + [len(p) for p in prompts])
        for a, e in zip(bounds[:-1], bounds[1:]):
            if e <= a:
                continue
            ids, sl = B.pkvt_tree_build(self.tree, prompts[a:e])
            full = np.full(int(tok_at[-1]), -1, np.int64)
            full[tok_at[a]:tok_at[e]] = sl
            src, dst = B.pkvt_tree_moves(self.tree)
            ids_parts.append(ids)
            builds.append((full, src, dst))
        self.seq_ids = np.concatenate(ids_parts).astype(np.int32)
        # each token's slot as its build returned it (later splits may move it)
        self.slots = np.max(np.stack([bl[0] for bl in builds]), axis=0)
        self.moves = sum(int(bl[1].size) for bl in builds)
        assert self.slots.shape[0] == total_tokens
        pool_elems = B.pkvt_pool_bytes(w.h, w.d, w.c, pool_chunks) // 2
        self.k_pools: List = []
        self.v_pools: List = []
        stream = torch.cuda.current_stream().cuda_stream
        gen = None
        if device_random_seed is not None or extra_layers_seed is not None:
            gen = torch.Generator(device=device)
            gen.manual_seed(device_random_seed if device_random_seed is not None else extra_layers_seed)
        for layer in range(self.layers):
            kp = torch.empty(pool_elems, dtype=torch.float16, device=device)
            vp = torch.empty(pool_elems, dtype=torch.float16, device=device)
            if device_random_seed is not None or (extra_layers_seed is not None and layer >= w.layers):
                kp.normal_(generator=gen)
                vp.normal_(generator=gen)
                self.k_pools.append(kp)
                self.v_pools.append(vp)
                continue
            for full, src, dst in builds:
                if src.size:
                    ms = torch.from_numpy(src).to(device)
                    md = torch.from_numpy(dst).to(device)
                    B.pkvt_kv_move(self.tree, kp.data_ptr(), vp.data_ptr(), ms.data_ptr(),
                                   md.data_ptr(), src.size, stream)
                    torch.cuda.synchronize()
                    del ms, md
                k_new, v_new, s_new = gather_new_tokens(w, full, layer)
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
        if device_random_seed is not None:
            self.q = torch.empty(w.q.shape, dtype=torch.float16, device=device).normal_(generator=gen)
        else:
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


class HostDecoder:
    """Tree side of decoding a trace (``workloads.DecodeTrace``).

    Per step: departures and arrivals of the step's joins (``pkvt_tree_remove``
    then ``pkvt_tree_build``), one ``pkvt_tree_append`` for the whole batch,
    and ``pkvt_plan`` for the rows' live sequences.  The library decides how
    much to redo (ChunkAttention page, Knowl 5, lazy context copy): only the
    length table when no chunk was opened; a patch of the rows' last items
    when appends opened new leaf chunks; a full rebuild after an arrival or
    departure.  Needs no GPU.  Host time per call is accumulated in ``us``
    (microseconds) and ``count`` under "plan_refresh", "plan_patch" and
    "plan_full"."""

    def __init__(self, tree: int, trace, seq_ids, **plan_kw):
        self.tree = tree
        self.tr = trace
        self.rows = np.array(seq_ids, dtype=np.int32)        # row -> live sequence id
        self.plan_kw = plan_kw
        self.us = {"join": 0.0, "append": 0.0, "plan_full": 0.0, "plan_patch": 0.0,
                   "plan_refresh": 0.0}
        self.count = {k: 0 for k in self.us}

    def _time(self, key, t0):
        import time
        self.us[key] += (time.perf_counter_ns() - t0) / 1e3
        self.count[key] += 1

    def joins(self, t: int):
        """Apply step t's departures/arrivals.  Returns [(join, prompt slots,
        (move src, move dst))]: under token matching an arrival may split a
        node, whose moved tokens' K/V the caller relocates before it writes
        the new tokens."""
        import time
        out = []
        for j in self.tr.joins_at(t):
            t0 = time.perf_counter_ns()
            B.pkvt_tree_remove(self.tree, int(self.rows[j.row]))
            ids, slots = B.pkvt_tree_build(self.tree, [self.tr.prompt_tokens(j)])
            moves = B.pkvt_tree_moves(self.tree)
            self.rows[j.row] = ids[0]
            self._time("join", t0)
            out.append((j, slots, moves))
        return out

    def append(self, t: int) -> np.ndarray:
        """Append step t's tokens; returns the slot of every row's new token."""
        import time
        t0 = time.perf_counter_ns()
        slots = B.pkvt_tree_append(self.tree, self.rows, self.tr.tokens[t])
        self._time("append", t0)
        return slots

    def plan(self):
        """(meta_bytes, workspace_bytes) of the plan for the rows' sequences."""
        import time
        t0 = time.perf_counter_ns()
        mb, wb = B.pkvt_plan(self.tree, self.rows, **self.plan_kw)
        el = time.perf_counter_ns() - t0
        kind = ("plan_refresh", "plan_patch", "plan_full")[B.pkvt_plan_last_update(self.tree)]
        self.us[kind] += el / 1e3
        self.count[kind] += 1
        return mb, wb


class DecodeLoop:
    """Decoding iterations over a ``DecodeSetup``, driven by a decode trace.

    Step t, as a model's attention layers would run it (ChunkAttention page,
    Knowl 1 and Knowl 5): the host applies the step's joins and appends one
    token per row; the new tokens' slots go to the device through a ring of
    pinned buffers; for every layer ``pkvt_kv_scatter`` writes the new K/V
    into that layer's pools; the plan is refreshed (rebuilt only after a
    structural change) and ``pkvt_plan_upload`` copies what changed; then
    ``pkvt_attn_decode`` runs for every layer with the step's queries,
    writing ``out[layer]``.  Nothing waits for the GPU except the pinned
    ring (a buffer is reused only after its copy has run).  The trace's
    per-step inputs live in device memory from construction on."""

    def __init__(self, ds: "DecodeSetup", trace, ring: int = 8, **plan_kw):
        torch = ds.torch
        self.torch = torch
        self.ds = ds
        self.tr = trace
        w = trace.base
        dev = ds.device
        if ds.layers > w.layers:
            raise ValueError("the trace has fewer layers than the setup")
        self.host = HostDecoder(ds.tree, trace, ds.seq_ids, **plan_kw)
        self.q = torch.from_numpy(trace.q).to(dev)
        self.k = [torch.from_numpy(trace.k[l]).to(dev) for l in range(ds.layers)]
        self.v = [torch.from_numpy(trace.v[l]).to(dev) for l in range(ds.layers)]
        self.join_kv = {}
        for j in trace.joins:
            self.join_kv[id(j)] = (
                [torch.from_numpy(np.ascontiguousarray(j.suffix.k[l])).to(dev) for l in range(ds.layers)],
                [torch.from_numpy(np.ascontiguousarray(j.suffix.v[l])).to(dev) for l in range(ds.layers)])
        self.out = torch.empty((ds.layers, w.b, w.h, w.d), dtype=torch.float16, device=dev)
        cap = max([w.b, w.c] + [len(j.suffix) + sum(len(w.segments[s]) for s in j.shared)
                                for j in trace.joins])
        self.ring = [(torch.empty(cap, dtype=torch.int64).pin_memory(),
                      torch.empty(cap, dtype=torch.int64, device=dev),
                      torch.cuda.Event()) for _ in range(ring)]
        self.ring_used = [False] * ring
        self.ring_at = 0
        self.regrow = 0
        self.us_total = 0.0
        self.steps_run = 0
        mb, wb = self.host.plan()
        self.meta = torch.empty(max(2 * mb, 1 << 16) // 4, dtype=torch.int32, device=dev)
        self.ws = torch.empty(max(2 * wb, 1 << 16) // 4, dtype=torch.float32, device=dev)
        self.meta_bytes = mb
        self.ws_bytes = wb
        B.pkvt_plan_upload(ds.tree, self.meta.data_ptr(), self.meta.numel() * 4,
                           torch.cuda.current_stream().cuda_stream)

    def _to_device(self, slots: np.ndarray):
        """Copy int64 slots to the device through the pinned ring."""
        k = self.ring_at
        self.ring_at = (k + 1) % len(self.ring)
        pin, dst, ev = self.ring[k]
        if self.ring_used[k]:
            ev.synchronize()
        n = slots.shape[0]
        pin[:n].numpy()[:] = slots
        dst[:n].copy_(pin[:n], non_blocking=True)
        ev.record()
        self.ring_used[k] = True
        return dst

    def _scatter(self, layer, d_slots, k_src, v_src, n, stream):
        ds = self.ds
        B.pkvt_kv_scatter(ds.tree, ds.k_pools[layer].data_ptr(), ds.v_pools[layer].data_ptr(),
                          d_slots.data_ptr(), k_src.data_ptr(), v_src.data_ptr(), n, stream)

    def _join_kv(self, j, slots, stream):
        """Write the K/V of a new sequence's prompt tokens that need storing:
        its suffix from device memory, and (when the kept prefix ends inside
        a chunk) the few prefix tokens that landed in a fresh chunk."""
        torch, ds, w = self.torch, self.ds, self.tr.base
        n_pre = sum(len(w.segments[s]) for s in j.shared)
        pre = slots[:n_pre]
        need = np.nonzero(pre >= 0)[0]
        if need.size:
            for l in range(ds.layers):
                kk = np.concatenate([w.segments[s].k[l] for s in j.shared])[need]
                vv = np.concatenate([w.segments[s].v[l] for s in j.shared])[need]
                kd = torch.from_numpy(np.ascontiguousarray(kk)).to(ds.device)
                vd = torch.from_numpy(np.ascontiguousarray(vv)).to(ds.device)
                d = self._to_device(pre[need])
                self._scatter(l, d, kd, vd, need.size, stream)
        suf = slots[n_pre:]
        if suf.size:
            d = self._to_device(suf)
            ks, vs = self.join_kv[id(j)]
            for l in range(ds.layers):
                self._scatter(l, d, ks[l], vs[l], suf.size, stream)

    def step(self, t: int, events=None):
        """Run decode step t.  ``events`` = (start, end) torch events recorded
        around the step's attention calls.  Host time of the step goes to
        ``us_total`` (microseconds); the part spent outside HostDecoder
        (copies, uploads, launches) is ``us_total`` minus the host's timers."""
        import time
        t_enter = time.perf_counter_ns()
        torch, ds = self.torch, self.ds
        stream = torch.cuda.current_stream().cuda_stream
        for j, slots, (src, dst) in self.host.joins(t):
            if src.size:
                d_src, d_dst = self._to_device(src), self._to_device(dst)
                for l in range(ds.layers):
                    B.pkvt_kv_move(ds.tree, ds.k_pools[l].data_ptr(), ds.v_pools[l].data_ptr(),
                                   d_src.data_ptr(), d_dst.data_ptr(), src.size, stream)
            self._join_kv(j, slots, stream)
        slots = self.host.append(t)
        b = self.tr.base.b
        if b <= B.PKVT_INLINE_SLOTS:
            # the slots travel in the scatter launches' arguments
            for l in range(ds.layers):
                B.pkvt_kv_scatter_host_slots(ds.tree, ds.k_pools[l].data_ptr(),
                                             ds.v_pools[l].data_ptr(), slots,
                                             self.k[l][t].data_ptr(), self.v[l][t].data_ptr(),
                                             stream)
        else:
            d = self._to_device(slots)
            for l in range(ds.layers):
                self._scatter(l, d, self.k[l][t], self.v[l][t], b, stream)
        mb, wb = self.host.plan()
        if mb > self.meta.numel() * 4 or wb > self.ws.numel() * 4:
            self.regrow += 1
            if mb > self.meta.numel() * 4:
                self.meta = torch.empty(2 * mb // 4, dtype=torch.int32, device=ds.device)
            if wb > self.ws.numel() * 4:
                self.ws = torch.empty(2 * wb // 4, dtype=torch.float32, device=ds.device)
        self.meta_bytes, self.ws_bytes = mb, wb
        B.pkvt_plan_upload(ds.tree, self.meta.data_ptr(), self.meta.numel() * 4, stream)
        if events is not None:
            events[0].record()
        q = self.q[t]
        for l in range(ds.layers):
            B.pkvt_attn_decode(ds.tree, self.meta.data_ptr(), q.data_ptr(),
                               ds.k_pools[l].data_ptr(), ds.v_pools[l].data_ptr(),
                               self.out[l].data_ptr(), self.ws.data_ptr() if wb else 0, wb,
                               ds.scale, stream)
        if events is not None:
            events[1].record()
        self.us_total += (time.perf_counter_ns() - t_enter) / 1e3
        self.steps_run += 1
        return self.out


def loop_pool_chunks(trace) -> int:
    """A pool size that a decode trace cannot exhaust: every base sequence's
    chunks as if nothing were shared, plus, for every row and every join,
    the chunks its appends and prompt could open (and one for the node it
    may split under token matching)."""
    w = trace.base
    c = w.c
    grow = trace.steps // c + 2
    n = sum(-(-w.seq_len(u) // c) for u in range(w.b)) + w.b * grow
    for j in trace.joins:
        n_pre = sum(len(w.segments[s]) for s in j.shared)
        n += -(-(n_pre + len(j.suffix)) // c) + grow + 1
    return n


class PrefillSetup:
    """A prefill batch (``workloads.PrefillBatch``) on the GPU: the resident
    prefix is inserted and its K/V written first, then the batch sequences
    arrive (``pkvt_tree_build``; their matched prefix chunks are shared), the
    new tokens' K/V are written by ``pkvt_kv_scatter``, and the prefill plan
    for rows q_from .. len - 1 of every sequence is built and uploaded."""

    def __init__(self, pb, layers: Optional[int] = None, device: str = "cuda",
                 phase1_chunks: int = 0, device_random_seed: Optional[int] = None,
                 pool_slack: int = 0, match: str = "chunks"):
        import torch
        self.torch = torch
        self.pb = pb
        w = pb.w
        self.w = w
        self.layers = w.layers if layers is None else layers
        self.device = device
        c = w.c
        pool_chunks = (sum(-(-len(w.segments[s]) // c) for s in pb.residents) +
                       sum(-(-w.seq_len(u) // c) for u in pb.seqs) + pool_slack)
        if match == "tokens":
            pool_chunks += len(pb.seqs)                  # a split per arrival at most
        self.tree = B.pkvt_tree_create(w.h, w.d, c, pool_chunks, match=match)
        stream = torch.cuda.current_stream().cuda_stream
        res_slots = np.zeros(0, np.int64)
        if pb.residents:
            self.resident_ids, res_slots = B.pkvt_tree_build(
                self.tree, [w.segments[s].tokens for s in pb.residents])
        self.seq_ids, slots = B.pkvt_tree_build(self.tree, [w.seq_tokens(u) for u in pb.seqs])
        move_src, move_dst = B.pkvt_tree_moves(self.tree)      # token matching: split tails
        pos = 0
        for u, a in zip(pb.seqs, pb.q_from):
            L = w.seq_len(u)
            s = slots[pos:pos + L]
            if not (np.all(s[:a] == -1) and np.all(s[a:] >= 0)):
                raise RuntimeError(f"sequence {u}: stored prefix does not end at q_from = {a}")
            pos += L
        pool_elems = B.pkvt_pool_bytes(w.h, w.d, c, pool_chunks) // 2
        gen = None
        if device_random_seed is not None:
            gen = torch.Generator(device=device)
            gen.manual_seed(device_random_seed)
        self.k_pools, self.v_pools = [], []
        for layer in range(self.layers):
            kp = torch.empty(pool_elems, dtype=torch.float16, device=device)
            vp = torch.empty(pool_elems, dtype=torch.float16, device=device)
            if gen is not None:
                kp.normal_(generator=gen)
                vp.normal_(generator=gen)
            else:
                writes = []
                at = 0
                for s in pb.residents:
                    seg = w.segments[s]
                    rs = res_slots[at:at + len(seg)]
                    at += len(seg)
                    need = np.nonzero(rs >= 0)[0]
                    writes.append((seg.k[layer][need], seg.v[layer][need], rs[need]))
                writes.append(None)                  # the batch's moves of stored tokens
                writes.append(gather_new_tokens(w, slots, layer))
                for item in writes:
                    if item is None:
                        if move_src.size:
                            ms = torch.from_numpy(move_src).to(device)
                            md = torch.from_numpy(move_dst).to(device)
                            B.pkvt_kv_move(self.tree, kp.data_ptr(), vp.data_ptr(), ms.data_ptr(),
                                           md.data_ptr(), move_src.size, stream)
                            torch.cuda.synchronize()
                        continue
                    k_new, v_new, s_new = item
                    if s_new.size == 0:
                        continue
                    kd = torch.from_numpy(np.ascontiguousarray(k_new)).to(device)
                    vd = torch.from_numpy(np.ascontiguousarray(v_new)).to(device)
                    sd = torch.from_numpy(np.ascontiguousarray(s_new, dtype=np.int64)).to(device)
                    B.pkvt_kv_scatter(self.tree, kp.data_ptr(), vp.data_ptr(), sd.data_ptr(),
                                      kd.data_ptr(), vd.data_ptr(), s_new.size, stream)
                    torch.cuda.synchronize()
            self.k_pools.append(kp)
            self.v_pools.append(vp)
        if gen is not None:
            self.q = torch.empty(pb.q.shape, dtype=torch.float16, device=device).normal_(generator=gen)
        else:
            self.q = torch.from_numpy(np.ascontiguousarray(pb.q)).to(device)
        self.out = torch.empty_like(self.q)
        self.scale = 1.0 / math.sqrt(w.d)
        self.replan(phase1_chunks)

    def replan(self, phase1_chunks: int = 0, workgroups: int = 0):
        torch = self.torch
        mb, wb = B.pkvt_prefill_plan(self.tree, self.seq_ids, self.pb.q_from,
                                     phase1_chunks=phase1_chunks, workgroups=workgroups)
        self.meta = torch.empty(max(mb // 4, 1), dtype=torch.int32, device=self.device)
        self.meta_bytes = mb
        self.ws = torch.empty(max(wb // 4, 1), dtype=torch.float32, device=self.device)
        self.ws_bytes = wb
        B.pkvt_prefill_upload(self.tree, self.meta.data_ptr(), mb,
                              torch.cuda.current_stream().cuda_stream)
        self.info = B.pkvt_prefill_info_get(self.tree)
        return self.info

    def run(self, layer: int = 0, out=None, stream: Optional[int] = None):
        torch = self.torch
        out = self.out if out is None else out
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        B.pkvt_prefill_attn(self.tree, self.meta.data_ptr(), self.q.data_ptr(),
                            self.k_pools[layer].data_ptr(), self.v_pools[layer].data_ptr(),
                            out.data_ptr(), self.ws.data_ptr(), self.ws_bytes, self.scale, stream)
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
