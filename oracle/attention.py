"""Attention oracle (fp64).  Test infrastructure only -- see the package header.

Sources (cited by page title and section):
  * "ChunkAttention: Efficient Self-Attention with Prefix-Aware KV Cache and
    Two-Phase Partition" (chapterpal digest), Knowl 3 (partial_attn /
    attn_reduce equations and the final division O = o / n) and Knowl 1 (a
    shared chunk is stored once).
  * "CachedAttention / AttentionStore" digest, section "Load-bearing
    equations": Attention(Q, K, V) = softmax(Q K^T / sqrt(d_K)) V, which
    fixes the 1/sqrt(d) score scale that the ChunkAttention equations leave
    out.

What the method computes, per sequence u of the decode batch and head h,
is the plain definition

    O[u, h] = sum_t softmax_t(s)_t * V_u[t, h],   s_t = q[u, h] . K_u[t, h] / sqrt(d)

over every token t currently stored for u (its root-to-leaf path).  The
two-phase partition reaches exactly this result up to rounding, because
attn_reduce is the exact online-softmax merge.  ``attention_batch`` is that
definition; ``partial_attn`` / ``attn_reduce`` restate the page's two
equations, and ``partitioned_attention`` uses them to assemble the result
from any cover of each context by disjoint pieces, so the tests can pin that
such a decomposition (the one the kernels rely on) agrees with it.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np


def materialize(w, u: int, layer: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """K_u, V_u as fp64 [L_u, h, d]: the segments on u's path, concatenated
    in path order (root prompt first, private suffix last).  fp16 -> fp64 is
    exact.  ``w`` is any object with ``segments`` (each with ``k``/``v``
    per-layer arrays [len, h, d]) and ``seq_paths``."""
    segs = [w.segments[s] for s in w.seq_paths[u]]
    K = np.concatenate([s.k[layer] for s in segs], axis=0).astype(np.float64)
    V = np.concatenate([s.v[layer] for s in segs], axis=0).astype(np.float64)
    return K, V


def attention_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V for every head.

    q [h, d]; K, V [L, h, d] (fp64).  Returns [h, d] fp64.  The max is
    subtracted before exponentiating (the usual stable evaluation; the
    softmax is unchanged by it)."""
    q = np.asarray(q, dtype=np.float64)
    s = np.einsum("hd,lhd->hl", q, K) * scale          # scores [h, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)                                  # [h, L]
    out = np.einsum("hl,lhd->hd", p, V)
    return out / p.sum(axis=1)[:, None]


def default_scale(d: int) -> float:
    """1/sqrt(d_K), the scale of the attention definition."""
    return 1.0 / math.sqrt(d)


def attention_batch(w, layer: int = 0, scale: float = None, seqs: Sequence[int] = None) -> np.ndarray:
    """O [b, h, d] fp64 for every sequence (or only ``seqs``; other rows NaN).

    One sequence is materialized at a time to bound memory."""
    b, h, d = w.q.shape
    if scale is None:
        scale = default_scale(d)
    out = np.full((b, h, d), np.nan, dtype=np.float64)
    for u in (range(b) if seqs is None else seqs):
        K, V = materialize(w, u, layer)
        out[u] = attention_one(w.q[u], K, V, scale)
    return out


# --------------------------------------------------------------------------
# Partitioned form (Knowl 3 equations), natural exp, fp64.
# --------------------------------------------------------------------------

def partial_attn(Qr: np.ndarray, Kc: np.ndarray, Vc: np.ndarray):
    """Knowl 3, partial_attn over one chunk for a block of query rows.

    Qr [R, d] (already multiplied by the score scale), Kc/Vc [n, d].
    W = Qr Kc^T; m = row max of W; E = exp(W - m); n = row sum of E;
    O = E Vc (unnormalized).  Returns (O [R, d], m [R], n [R])."""
    W = Qr @ Kc.T
    m = W.max(axis=1)
    E = np.exp(W - m[:, None])
    n = E.sum(axis=1)
    return E @ Vc, m, n


def attn_reduce(oC, mC, nC, ou, mu, nu):
    """Knowl 3, attn_reduce: merge a chunk's partial (oC, mC, nC) into the
    running accumulators (ou, mu, nu) of one sequence.

    x = exp(mC - max), y = exp(mu - max), o = x oC + y ou, n = x nC + y nu,
    m = max.  The accumulator's initial state (o = 0, m = -inf, n = 0) is the
    identity of this merge; exp(-inf - (-inf)) is undefined, so a side whose
    m is -inf contributes nothing and is skipped explicitly."""
    if mC == -math.inf:
        return ou, mu, nu
    if mu == -math.inf:
        return np.array(oC, dtype=np.float64), mC, nC
    M = max(mC, mu)
    x = math.exp(mC - M)
    y = math.exp(mu - M)
    return x * oC + y * ou, M, x * nC + y * nu


def partitioned_attention(w, pieces: Sequence[Sequence[Tuple[int, int, int]]], layer: int = 0,
                          scale: float = None) -> np.ndarray:
    """Attention assembled from partials over pieces of each context, fp64.

    Knowl 3's two equations make attention over a key set decomposable: the
    partial (o, m, n) of any subset of the keys carries everything needed,
    and attn_reduce of the partials of disjoint subsets is the partial of
    their union.  So for any cover of u's keys by disjoint pieces, folding
    the pieces' partials in any order and dividing o by n gives the plain
    result.  ``pieces[u]`` lists u's pieces in the order they are folded;
    a piece (src, lo, hi) stands for keys lo .. hi-1 of sequence ``src``'s
    materialised K/V.  With src = u and any partition of [0, L_u) the result
    equals ``attention_batch``; a piece taken from another sequence models a
    stored chunk that the tree claims both sequences hold (Knowl 1: a shared
    chunk is stored once), so a wrong claim changes the result."""
    b, h, d = w.q.shape
    if scale is None:
        scale = default_scale(d)
    mats: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
    out = np.empty((b, h, d), dtype=np.float64)
    for u in range(b):
        for hh in range(h):
            qs = w.q[u, hh].astype(np.float64)[None, :] * scale
            o, m, n = np.zeros(d), -math.inf, 0.0
            for src, lo, hi in pieces[u]:
                if src not in mats:
                    mats[src] = materialize(w, src, layer)
                K, V = mats[src]
                Op, mp, np_ = partial_attn(qs, K[lo:hi, hh], V[lo:hi, hh])
                o, m, n = attn_reduce(Op[0], mp[0], np_[0], o, m, n)
            out[u, hh] = o / n
    return out


def pieces_from_labels(chunk_labels: List[np.ndarray], c: int, lens: Sequence[int]):
    """The chunk pieces of every context under a sharing map: chunk k of u
    is keys k*c .. min((k+1)*c, L) of the first sequence (in index order)
    whose path holds the same label -- the one stored copy of a shared
    chunk.  Returns ``pieces`` for ``partitioned_attention`` (path order)."""
    holder: Dict[int, Tuple[int, int]] = {}
    for u, labs in enumerate(chunk_labels):
        for k, lab in enumerate(labs):
            holder.setdefault(int(lab), (u, k))
    out = []
    for u, labs in enumerate(chunk_labels):
        row = []
        for lab in labs:
            src, k = holder[int(lab)]
            row.append((src, k * c, min((k + 1) * c, int(lens[src]))))
        out.append(row)
    return out


# --------------------------------------------------------------------------
# Prefill: many new query rows per sequence, causal.
# --------------------------------------------------------------------------

def prefill_rows(w, seqs: Sequence[int], q_from: Sequence[int]) -> List[Tuple[int, int]]:
    """The (sequence, position) of every prefill query row, in row order:
    for each u of ``seqs`` in order, positions q_from[i] .. L_u - 1."""
    rows = []
    for u, a in zip(seqs, q_from):
        rows += [(int(u), p) for p in range(int(a), w.seq_len(int(u)))]
    return rows


def prefill_attention(w, seqs: Sequence[int], q_from: Sequence[int], q: np.ndarray,
                      layer: int = 0, scale: float = None, rows: Sequence[int] = None) -> np.ndarray:
    """Causal attention of prefill query rows, fp64.

    A new token at position p of sequence u attends to u's tokens 0..p: the
    keys already stored before it (a matched shared prefix, or earlier
    pieces of a chunked prompt) and the new tokens up to itself (causal
    visibility; ChunkAttention page, Knowl 1 arrival; the chunked-prefill
    page, sections 1-2: append-only KV and the causal mask make feeding a
    prompt in pieces exact).  ``q`` [R, h, d] holds the rows of
    ``prefill_rows(w, seqs, q_from)``; returns O [R, h, d] (only ``rows``
    filled when given, NaN elsewhere)."""
    R, h, d = q.shape
    if scale is None:
        scale = default_scale(d)
    meta = prefill_rows(w, seqs, q_from)
    assert len(meta) == R
    out = np.full((R, h, d), np.nan, dtype=np.float64)
    want = set(range(R)) if rows is None else set(int(r) for r in rows)
    cache_u, KV = None, None
    for r, (u, p) in enumerate(meta):
        if r not in want:
            continue
        if u != cache_u:
            KV, cache_u = materialize(w, u, layer), u
        K, V = KV
        out[r] = attention_one(q[r], K[:p + 1], V[:p + 1], scale)
    return out
