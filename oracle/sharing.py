"""Sharing-map oracle.  Test infrastructure only -- see the package header.

Source: "ChunkAttention: Efficient Self-Attention with Prefix-Aware KV Cache
and Two-Phase Partition" (chapterpal digest), Knowl 1 (the prefix-aware KV
cache: fixed-size chunks of c tokens as tree nodes, one root-to-leaf path per
sequence, arrival / decoding / departure rules, pool allocator) and Knowl 4
(sharing ratio, capacity multiplier, fragmentation bound).

Readings of the page used here (the page leaves them open):
  * Matching is whole-chunk and starts at token 0: a chunk is shared only
    when it is full (c tokens) and the entire token prefix up to and
    including it is identical.  A partial tail chunk is always private, and
    a decode append never writes into a shared chunk.
  * A chunk that becomes full through decode appends is an ordinary node
    from then on and can be matched by later arrivals; nodes are never
    merged or de-duplicated.  When several live children of one node carry
    the same c tokens, a lookup takes the earliest created one.

Token-granular variant (TokenSharingModel; the page's nodes are whole
chunks, this is the variant that shares a prefix which ends inside a chunk):
  * a node holds 1..c tokens at the start of its chunk;
  * an arrival descends from the root, at each node into the child whose
    tokens share the longest common prefix with the rest of the prompt
    (ties: the earliest created); a child matched only in its first t
    tokens is split: it keeps those t tokens and a new node, inserted below
    it and above its old children, takes the rest (their K/V move to the new
    node's chunk); the unmatched rest of the prompt becomes a new branch;
  * a decode append writes into the sequence's leaf only while that leaf is
    partial, private and childless; otherwise it opens a new leaf chunk (a
    shared or split chunk is never written again);
  * nodes are never merged.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np


def chunk_labels(token_seqs: Sequence[Sequence[int]], c: int) -> List[np.ndarray]:
    """Canonical chunk identities for a tree built by inserting the given
    sequences in order (no decode appends, no removals).

    Definition: chunk k of sequences u and v is the same stored chunk iff
    both are full and tokens_u[0:(k+1)c] == tokens_v[0:(k+1)c].  A partial
    tail chunk has an identity of its own.  Labels are numbered by first
    appearance, scanning sequences in order and chunk positions ascending.
    """
    first: Dict[tuple, int] = {}
    out: List[np.ndarray] = []
    for u, toks in enumerate(token_seqs):
        toks = [int(t) for t in toks]
        n = len(toks)
        labs = []
        for k in range((n + c - 1) // c):
            if (k + 1) * c <= n:
                key = ("full", tuple(toks[:(k + 1) * c]))
            else:
                key = ("tail", u)
            if key not in first:
                first[key] = len(first)
            labs.append(first[key])
        out.append(np.asarray(labs, dtype=np.int32))
    return out


def canonicalize(paths: Sequence[Sequence[int]]) -> List[np.ndarray]:
    """Renumber arbitrary chunk ids by first appearance (sequences in order,
    positions ascending), so two sharing maps can be compared as arrays."""
    first: Dict[int, int] = {}
    out = []
    for p in paths:
        labs = []
        for x in p:
            x = int(x)
            if x not in first:
                first[x] = len(first)
            labs.append(first[x])
        out.append(np.asarray(labs, dtype=np.int32))
    return out


def coverage(labels: Sequence[np.ndarray]) -> Dict[int, List[int]]:
    """label -> sorted list of the sequences whose path contains it."""
    cov: Dict[int, set] = {}
    for u, labs in enumerate(labels):
        for x in labs:
            cov.setdefault(int(x), set()).add(u)
    return {k: sorted(v) for k, v in cov.items()}


# --------------------------------------------------------------------------
# Knowl 4 closed forms.
# --------------------------------------------------------------------------

def sharing_ratio(n_s: float, n_p: float, n_c: float) -> float:
    """r = n_s / (n_p + n_c)."""
    return n_s / (n_p + n_c)


def capacity_multiplier(r: float) -> float:
    """Approximate gain in concurrent sequences from sharing: 1 / (1 - r)."""
    return 1.0 / (1.0 - r)


def fragmentation_bound(c: int, n: int) -> float:
    """Upper bound on the fraction of a sequence's leaf-chunk storage lost to
    internal fragmentation: (c - 1) / n."""
    return (c - 1) / n


# --------------------------------------------------------------------------
# Reference model of arrival / decode append / departure (Knowl 1).
# --------------------------------------------------------------------------

class _Node:
    __slots__ = ("nid", "parent", "tokens", "children", "refs")

    def __init__(self, nid: int, parent: Optional["_Node"], tokens: List[int]):
        self.nid = nid
        self.parent = parent
        self.tokens = tokens
        self.children: List["_Node"] = []   # creation order
        self.refs: set = set()


class SharingModel:
    """A plain prefix-tree model of which chunks are stored and shared.

    Node ids are creation counters and are never reused, so they are
    identities, not storage addresses.  ``paths()`` gives every live
    sequence's node ids root to leaf; ``canonicalize`` turns them into labels
    comparable with any other implementation's chunk ids."""

    def __init__(self, c: int):
        self.c = c
        self.root = _Node(-1, None, [])
        self.next_id = 0
        self.seqs: Dict[int, List[_Node]] = {}
        self.next_seq = 0

    def _new(self, parent: _Node, toks: List[int]) -> _Node:
        n = _Node(self.next_id, parent, toks)
        self.next_id += 1
        parent.children.append(n)
        return n

    def _find_full(self, parent: _Node, key: List[int]) -> Optional[_Node]:
        for ch in parent.children:          # creation order: earliest first
            if len(ch.tokens) == self.c and ch.tokens == key:
                return ch
        return None

    def insert(self, tokens: Sequence[int]) -> int:
        """Sequence arrival: share matching full chunks from token 0, then
        store the rest as a new branch (the tail chunk may be partial)."""
        toks = [int(t) for t in tokens]
        if not toks:
            raise ValueError("empty sequence")
        sid = self.next_seq
        self.next_seq += 1
        node = self.root
        path: List[_Node] = []
        pos = 0
        matching = True
        while pos < len(toks):
            piece = toks[pos:pos + self.c]
            nxt = self._find_full(node, piece) if (matching and len(piece) == self.c) else None
            if nxt is None:
                matching = False
                nxt = self._new(node, piece)
            path.append(nxt)
            node = nxt
            pos += len(piece)
        for n in path:
            n.refs.add(sid)
        self.seqs[sid] = path
        return sid

    def append(self, sid: int, token: int) -> None:
        """Decode step: write into the leaf until it is full, then start a
        new private leaf."""
        path = self.seqs[sid]
        leaf = path[-1]
        if len(leaf.tokens) < self.c:
            assert leaf.refs == {sid}, "a partial leaf is always private"
            leaf.tokens.append(int(token))
        else:
            n = self._new(leaf, [int(token)])
            n.refs.add(sid)
            path.append(n)

    def remove(self, sid: int) -> None:
        """Departure: drop the sequence from its path; chunks no live
        sequence uses any more are freed and their nodes pruned."""
        path = self.seqs.pop(sid)
        for n in reversed(path):
            n.refs.discard(sid)
            if not n.refs:
                assert not n.children
                n.parent.children.remove(n)

    # ---- views -----------------------------------------------------------
    def live(self) -> List[int]:
        return sorted(self.seqs)

    def paths(self) -> List[List[int]]:
        return [[n.nid for n in self.seqs[s]] for s in self.live()]

    def refcounts(self) -> Dict[int, int]:
        out: Dict[int, int] = {}
        for s in self.live():
            for n in self.seqs[s]:
                out[n.nid] = len(n.refs)
        return out

    def used_chunks(self) -> int:
        return len({n.nid for s in self.live() for n in self.seqs[s]})

    def seq_len(self, sid: int) -> int:
        return sum(len(n.tokens) for n in self.seqs[sid])


# --------------------------------------------------------------------------
# Token-granular variant (see the module header).
# --------------------------------------------------------------------------

def common_prefix_len(a: Sequence[int], b: Sequence[int]) -> int:
    """Length of the longest common prefix of two token lists."""
    n = min(len(a), len(b))
    k = 0
    while k < n and int(a[k]) == int(b[k]):
        k += 1
    return k


def distinct_prefixes(token_seqs: Sequence[Sequence[int]]) -> int:
    """Number of distinct non-empty token prefixes over the sequences: the
    tokens a token-granular tree stores when every shared prefix is stored
    once."""
    seen = set()
    for toks in token_seqs:
        t = tuple(int(x) for x in toks)
        for k in range(1, len(t) + 1):
            seen.add(t[:k])
    return len(seen)


class TokenSharingModel(SharingModel):
    """SharingModel with token-granular matching and node splitting."""

    def _split(self, node: _Node, t: int) -> _Node:
        """Keep the first t tokens in node; a new node below it takes the
        rest and node's children; every sequence through node now also
        passes through the new node."""
        tail = _Node(self.next_id, node, node.tokens[t:])
        self.next_id += 1
        tail.children = node.children
        for ch in tail.children:
            ch.parent = tail
        node.tokens = node.tokens[:t]
        node.children = [tail]
        tail.refs = set(node.refs)
        for sid in node.refs:
            path = self.seqs[sid]
            i = path.index(node)
            path.insert(i + 1, tail)
        return tail

    def insert(self, tokens: Sequence[int]) -> int:
        toks = [int(t) for t in tokens]
        if not toks:
            raise ValueError("empty sequence")
        sid = self.next_seq
        self.next_seq += 1
        node = self.root
        path: List[_Node] = []
        pos = 0
        while pos < len(toks):
            best, best_len = None, 0
            for ch in node.children:            # creation order: earliest wins ties
                k = common_prefix_len(ch.tokens, toks[pos:])
                if k > best_len:
                    best, best_len = ch, k
            if best is None:
                break
            if best_len < len(best.tokens):
                self._split(best, best_len)
            path.append(best)
            node = best
            pos += best_len
        while pos < len(toks):
            piece = toks[pos:pos + self.c]
            node = self._new(node, piece)
            path.append(node)
            pos += len(piece)
        for n in path:
            n.refs.add(sid)
        self.seqs[sid] = path
        return sid

    def append(self, sid: int, token: int) -> None:
        path = self.seqs[sid]
        leaf = path[-1]
        if len(leaf.tokens) < self.c and leaf.refs == {sid} and not leaf.children:
            leaf.tokens.append(int(token))
        else:
            n = self._new(leaf, [int(token)])
            n.refs.add(sid)
            path.append(n)

    def node_tokens(self, sid: int) -> List[List[int]]:
        """The sequence's path as the token lists of its nodes."""
        return [list(n.tokens) for n in self.seqs[sid]]
