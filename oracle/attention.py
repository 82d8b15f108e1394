"""Attention oracle (fp64).  Test infrastructure only -- see the package header.

Sources (cited by page title and section):
  * "ChunkAttention: Efficient Self-Attention with Prefix-Aware KV Cache and
    Two-Phase Partition" (chapterpal digest), Knowl 2 (the two-phase
    partition algorithm) and Knowl 3 (partial_attn / attn_reduce equations
    and the final division O = o / n).
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
definition; ``partial_attn`` / ``attn_reduce`` / ``tpp_attention`` restate
the page's partitioned form so the tests can pin that it agrees.
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
# Partitioned form (Knowl 3 equations, Knowl 2 algorithm), natural exp, fp64.
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


def tpp_attention(w, chunk_labels: List[np.ndarray], c: int, layer: int = 0,
                  scale: float = None, order: str = "path", rng=None,
                  min_share: int = 2) -> np.ndarray:
    """The two-phase partition of Knowl 2, in fp64, on the oracle's own chunks.

    ``chunk_labels[u][k]`` identifies chunk k of sequence u (equal labels =
    the same stored chunk, as produced by ``oracle.sharing.chunk_labels``).
    Phase 1 visits every chunk covered by at least ``min_share`` sequences
    once, running partial_attn for all covering query rows together.  Phase
    2 folds, per sequence, those partials and then the sequence's own chunks
    through attn_reduce, and divides.  ``order`` selects the fold order
    ("path", "reverse" or "random") -- the merge is order-independent up to
    rounding, which the tests check.  The K/V of a shared chunk is read from
    the first covering sequence, so a wrong sharing map would change the
    result."""
    b, h, d = w.q.shape
    if scale is None:
        scale = default_scale(d)
    mats = [materialize(w, u, layer) for u in range(b)]
    cover: Dict[int, List[Tuple[int, int]]] = {}
    for u, labs in enumerate(chunk_labels):
        for k, lab in enumerate(labs):
            cover.setdefault(int(lab), []).append((u, k))
    out = np.empty((b, h, d), dtype=np.float64)
    for hh in range(h):
        # Phase 1: chunk-first over shared chunks.
        shared_parts: Dict[int, Dict[int, tuple]] = {}
        for lab, users in cover.items():
            if len(users) < min_share:
                continue
            u0, k0 = users[0]
            K, V = mats[u0]
            sl = slice(k0 * c, min((k0 + 1) * c, K.shape[0]))
            rows = np.stack([w.q[u, hh].astype(np.float64) * scale for u, _ in users])
            O, m, n = partial_attn(rows, K[sl, hh], V[sl, hh])
            shared_parts[lab] = {u: (O[i], m[i], n[i]) for i, (u, _) in enumerate(users)}
        # Phase 2: sequence-first.
        for u in range(b):
            K, V = mats[u]
            qs = w.q[u, hh].astype(np.float64)[None, :] * scale
            parts = []
            for k, lab in enumerate(chunk_labels[u]):
                lab = int(lab)
                if lab in shared_parts:
                    parts.append(shared_parts[lab][u])
                else:
                    sl = slice(k * c, min((k + 1) * c, K.shape[0]))
                    O, m, n = partial_attn(qs, K[sl, hh], V[sl, hh])
                    parts.append((O[0], m[0], n[0]))
            if order == "reverse":
                parts = parts[::-1]
            elif order == "random":
                perm = (rng or np.random.default_rng(0)).permutation(len(parts))
                parts = [parts[i] for i in perm]
            o, m, n = np.zeros(d), -math.inf, 0.0
            for oC, mC, nC in parts:
                o, m, n = attn_reduce(oC, mC, nC, o, m, n)
            out[u, hh] = o / n
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
