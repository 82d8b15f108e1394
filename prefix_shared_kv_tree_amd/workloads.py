"""Seeded synthetic decode workloads for prefix-shared KV attention.

This module only draws inputs. It holds none of the attention arithmetic and
none of the tree logic, so both the fp64 oracle (through the tests) and the
HIP path consume exactly the same arrays.

A workload is a set of token *segments* (a shared root prompt, a shared
branch, a private suffix...) and, for every sequence of the decode batch, the
list of segments its context is made of, in order.  Each segment carries its
own K and V values, drawn once, so a segment shared by several sequences is
literally the same array for all of them.  Shapes follow the microkernel
benchmark of the ChunkAttention page (Knowl 6: one decoded token per
sequence, h heads, head_dim d, chunk size c, fp16 Q/K/V); values are N(0,1)
drawn in float32 and rounded to fp16 (round-to-nearest-even).

Draw order for a named config (all from one numpy PCG64 generator seeded
with ``1000 + config index``):
  1. structure parameters (only the long-prompt config: the private suffix
     lengths, ``integers(256, 1025)`` per sequence),
  2. token ids of every segment, in segment order, uniform in [0, 32000),
  3. Q as a [b, h, d] block,
  4. for each layer, for each segment in order: K [len, h, d] then V.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

VOCAB = 32000

#: Names of the seeded configurations, in index order (seed = 1000 + index).
CONFIG_NAMES = ("tiny", "c2", "c3", "c4", "c5")
#: Diagnostic workloads (not among the benchmark configurations); their seeds
#: continue the index order.
DIAGNOSTIC_NAMES = ("phase1",)

CONFIG_DESCRIPTIONS = {
    "tiny": "4 decode queries, 2 heads, head_dim 64, chunk 16; one shared "
            "64-token prefix plus a private 32-token suffix per sequence",
    "c2": "32 heads, head_dim 128, chunk 64; batch 32 sharing a 1024-token "
          "prefix, private 512-token suffix each",
    "c3": "32 heads, head_dim 128, chunk 64; batch 64 sharing a 4096-token "
          "prefix, private suffix lengths uniform in [256, 1024]",
    "c4": "32 heads, head_dim 128, chunk 64; 2 roots x 2048 tokens (32 seqs "
          "each), 4 branches x 512 tokens per root (8 seqs each), private "
          "256-token suffixes; batch 64",
    "c5": "32 heads, head_dim 128, chunk 64; batch 64, each over its own "
          "private 2048-token context (nothing shared)",
    "phase1": "diagnostic: 32 heads, head_dim 128, chunk 64; batch 64 whose whole "
              "context is one shared 4096-token prefix (all work is chunk-first)",
}


@dataclasses.dataclass
class Segment:
    """A run of consecutive context tokens with its per-layer K and V."""
    tokens: np.ndarray                 # int32 [L]
    k: List[np.ndarray]                # per layer: float16 [L, h, d]
    v: List[np.ndarray]                # per layer: float16 [L, h, d]

    def __len__(self) -> int:
        return int(self.tokens.shape[0])


@dataclasses.dataclass
class Workload:
    name: str
    h: int
    d: int
    c: int
    segments: List[Segment]
    seq_paths: List[List[int]]         # per sequence: segment indices, in order
    q: np.ndarray                      # float16 [b, h, d]
    layers: int = 1

    @property
    def b(self) -> int:
        return len(self.seq_paths)

    def seq_tokens(self, u: int) -> np.ndarray:
        return np.concatenate([self.segments[s].tokens for s in self.seq_paths[u]])

    def seq_len(self, u: int) -> int:
        return int(sum(len(self.segments[s]) for s in self.seq_paths[u]))

    def all_seq_tokens(self) -> List[np.ndarray]:
        return [self.seq_tokens(u) for u in range(self.b)]


def _normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) drawn as float32, rounded to fp16. Drawn in slabs to bound memory."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float16)
    if out.size == 0:
        return out
    flat = out.reshape(shape[0], -1)
    row = flat.shape[1]
    step = max(1, (1 << 24) // max(row, 1))
    for i in range(0, shape[0], step):
        j = min(shape[0], i + step)
        flat[i:j] = rng.standard_normal((j - i, row), dtype=np.float32).astype(np.float16)
    return out


def _finish(name, rng, h, d, c, seg_lens, seq_paths, layers, token_fn=None,
            with_kv: bool = True) -> Workload:
    tokens = []
    for L in seg_lens:
        if token_fn is None:
            tokens.append(rng.integers(0, VOCAB, size=L, dtype=np.int64).astype(np.int32))
        else:
            tokens.append(token_fn(L))
    b = len(seq_paths)
    q = _normal_f16(rng, (b, h, d))
    segs = [Segment(tokens=t, k=[], v=[]) for t in tokens]
    for _ in range(layers if with_kv else 0):
        for s in segs:
            s.k.append(_normal_f16(rng, (len(s), h, d)))
            s.v.append(_normal_f16(rng, (len(s), h, d)))
    return Workload(name=name, h=h, d=d, c=c, segments=segs,
                    seq_paths=[list(p) for p in seq_paths], q=q, layers=layers)


def make_config(name: str, layers: int = 1, seed: Optional[int] = None,
                with_kv: bool = True) -> Workload:
    """Build one of the named configurations (see CONFIG_DESCRIPTIONS).

    ``with_kv=False`` skips the K/V draws (they come last, so tokens and Q
    are unchanged) for tests that only need the token structure."""
    idx = (CONFIG_NAMES + DIAGNOSTIC_NAMES).index(name)
    rng = np.random.Generator(np.random.PCG64(1000 + idx if seed is None else seed))
    if name == "tiny":
        b, h, d, c = 4, 2, 64, 16
        seg_lens = [64] + [32] * b
        paths = [[0, 1 + u] for u in range(b)]
        return _finish(name, rng, h, d, c, seg_lens, paths, layers, with_kv=with_kv)
    h, d, c = 32, 128, 64
    if name == "c2":
        b = 32
        seg_lens = [1024] + [512] * b
        paths = [[0, 1 + u] for u in range(b)]
    elif name == "c3":
        b = 64
        priv = rng.integers(256, 1025, size=b)
        seg_lens = [4096] + [int(x) for x in priv]
        paths = [[0, 1 + u] for u in range(b)]
    elif name == "c4":
        b = 64
        # segments: 2 roots, 8 branches (root r owns branches 2 + 4r .. 2 + 4r + 3), 64 privates
        seg_lens = [2048, 2048] + [512] * 8 + [256] * b
        paths = []
        for u in range(b):
            root = u // 32
            branch = 2 + 4 * root + (u // 8) % 4
            paths.append([root, branch, 10 + u])
    elif name == "c5":
        b = 64
        seg_lens = [2048] * b
        paths = [[u] for u in range(b)]
    elif name == "phase1":
        b = 64
        seg_lens = [4096]
        paths = [[0] for _ in range(b)]
    else:  # pragma: no cover
        raise ValueError(name)
    return _finish(name, rng, h, d, c, seg_lens, paths, layers, with_kv=with_kv)


def random_tree(seed: int, h: int = 2, d: int = 16, c: int = 4, max_b: int = 6,
                max_len: int = 80, vocab: int = VOCAB, layers: int = 1,
                unaligned: bool = True, min_b: int = 1) -> Workload:
    """A small random prefix forest with ragged lengths.

    Each new sequence either starts a fresh root (probability 0.2) or picks a
    random earlier sequence and a random cut point, reuses that sequence's
    first ``cut`` tokens (the same segments, hence the same K/V values) and
    appends a fresh suffix.  With ``unaligned`` the cut is any token
    position, so chunk boundaries and segment boundaries need not coincide.
    A small ``vocab`` makes accidental full-chunk matches between unrelated
    token runs likely; use it only for tree tests, since attention parity
    additionally needs equal token prefixes to carry equal K/V values.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    b = int(rng.integers(min_b, max_b + 1))
    seg_tokens: List[np.ndarray] = []
    paths: List[List[int]] = []

    def new_seg(toks):
        seg_tokens.append(np.asarray(toks, dtype=np.int32))
        return len(seg_tokens) - 1

    def fresh(L):
        return new_seg(rng.integers(0, vocab, size=L, dtype=np.int64))

    for u in range(b):
        if u == 0 or rng.random() < 0.2:
            paths.append([fresh(int(rng.integers(1, max_len + 1)))])
            continue
        parent = list(paths[int(rng.integers(0, u))])
        plen = sum(len(seg_tokens[s]) for s in parent)
        cut = int(rng.integers(0, plen + 1))
        if not unaligned:
            cut -= cut % c
        path: List[int] = []
        acc = 0
        split = None
        for s in parent:
            L = len(seg_tokens[s])
            if acc + L <= cut:
                path.append(s)
                acc += L
                continue
            take = cut - acc
            if take > 0:
                split = (s, take)
            break
        if split is not None:
            s, take = split
            head = new_seg(seg_tokens[s][:take])
            tail = new_seg(seg_tokens[s][take:])
            for p in paths:
                if s in p:
                    i = p.index(s)
                    p[i:i + 1] = [head, tail]
            path.append(head)
            acc += take
        extra = int(rng.integers(0 if acc > 0 else 1, max(2, max_len - acc + 1)))
        if extra > 0:
            path.append(fresh(extra))
        paths.append(path)
    used = sorted({s for p in paths for s in p})
    remap = {s: i for i, s in enumerate(used)}
    tok_list = [seg_tokens[s] for s in used]
    paths = [[remap[s] for s in p] for p in paths]
    it = iter(tok_list)
    return _finish(f"random{seed}", rng, h, d, c, [len(t) for t in tok_list], paths,
                   layers, token_fn=lambda L: next(it))


def one_prefix(seed: int, b: int, prefix: int, suffix, h: int = 2, d: int = 64, c: int = 16,
               layers: int = 1, with_kv: bool = True) -> Workload:
    """b sequences that share one prefix of ``prefix`` tokens, each followed
    by a private suffix (``suffix`` tokens, or a list of b lengths)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    suf = [int(suffix)] * b if np.isscalar(suffix) else [int(x) for x in suffix]
    seg_lens = ([prefix] if prefix > 0 else []) + suf
    if prefix > 0:
        paths = [[0, 1 + u] if suf[u] > 0 else [0] for u in range(b)]
    else:
        paths = [[u] for u in range(b)]
    return _finish(f"one_prefix{b}x{prefix}", rng, h, d, c, seg_lens, paths, layers,
                   with_kv=with_kv)


def layered_tree(seed: int, b: int, n_roots: int, h: int = 2, d: int = 64, c: int = 16,
                 max_chunks: int = 3, layers: int = 1) -> Workload:
    """A three-level forest with wide nodes: the b sequences are split into
    n_roots contiguous groups that each share a root segment, every group
    into 1..4 contiguous branches that each share a branch segment, and every
    sequence ends in a private suffix.  Segment lengths are random: roots
    1..max_chunks whole chunks, branches 0..max_chunks chunks plus sometimes a
    partial chunk (whose tail then cannot be shared), suffixes 1..2c tokens."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seg_lens: List[int] = []
    paths: List[List[int]] = []
    bounds = np.linspace(0, b, n_roots + 1).astype(int)
    for r in range(n_roots):
        lo, hi = int(bounds[r]), int(bounds[r + 1])
        if hi <= lo:
            continue
        seg_lens.append(c * int(rng.integers(1, max_chunks + 1)))
        root = len(seg_lens) - 1
        n_br = int(rng.integers(1, 5))
        cuts = sorted(set([lo, hi] + [int(x) for x in rng.integers(lo, hi, size=n_br - 1)]))
        for a, e in zip(cuts[:-1], cuts[1:]):
            L = c * int(rng.integers(0, max_chunks + 1))
            if rng.random() < 0.3:
                L += int(rng.integers(1, c))
            br = None
            if L > 0:
                seg_lens.append(L)
                br = len(seg_lens) - 1
            for _ in range(a, e):
                seg_lens.append(int(rng.integers(1, 2 * c + 1)))
                paths.append([root] + ([br] if br is not None else []) + [len(seg_lens) - 1])
    return _finish(f"layered{b}", rng, h, d, c, seg_lens, paths, layers)


def unshare(w: Workload, token_offset: int = 1 << 20) -> Workload:
    """Same K/V values, but every sequence gets private copies of its segments
    under distinct token ids, so nothing can be shared by a prefix tree.  The
    attention result per sequence is unchanged by construction."""
    segs: List[Segment] = []
    paths: List[List[int]] = []
    for u, p in enumerate(w.seq_paths):
        np_ = []
        for s in p:
            src = w.segments[s]
            segs.append(Segment(tokens=src.tokens + np.int32(token_offset * (u + 1)),
                                k=src.k, v=src.v))
            np_.append(len(segs) - 1)
        paths.append(np_)
    return Workload(name=w.name + "-unshared", h=w.h, d=w.d, c=w.c, segments=segs,
                    seq_paths=paths, q=w.q, layers=w.layers)


def unique_segment_starts(w: Workload, base: int = VOCAB) -> Workload:
    """Give every segment a first token id that no other segment starts with
    (ids from ``base`` on), so that two contexts share exactly their common
    leading segments however finely a prefix tree matches tokens.  K/V values
    belong to segments, so token-granular sharing then never joins tokens
    with different K/V.  Lengths, K/V and Q are unchanged."""
    segs = []
    for i, sg in enumerate(w.segments):
        t = sg.tokens.copy()
        if t.size:
            t[0] = base + i
        segs.append(Segment(tokens=t, k=sg.k, v=sg.v))
    return Workload(name=w.name, h=w.h, d=w.d, c=w.c, segments=segs,
                    seq_paths=[list(p) for p in w.seq_paths], q=w.q, layers=w.layers)


def unique_tokens(w: Workload) -> int:
    """Number of distinct token positions when every full-chunk prefix is
    stored once: this is the count of *stored* KV rows, used for the
    effective-bytes metric.  Computed from segment structure only for the
    named configs, whose shared boundaries are chunk-aligned."""
    return int(sum(len(s) for s in w.segments))


def logical_tokens(w: Workload) -> int:
    return int(sum(w.seq_len(u) for u in range(w.b)))


# ---- decode traces -------------------------------------------------------------
#
# A decode trace drives a batch through T decoding iterations (ChunkAttention
# page, Knowl 1: each iteration appends one token per sequence to its leaf
# chunk; sequences leave and new ones arrive while decoding goes on).  Row r
# of the batch is one slot of the serving batch: at step t it holds one live
# sequence, whose query is q[t, r] and whose new token (id, and K/V of every
# layer) is tokens[t, r], k[layer][t, r], v[layer][t, r].  A join at step t
# replaces the sequence of its row before that step's append: the old
# sequence departs, and a new one arrives whose prompt is the old one's
# shared segments (every segment of its base path but the last) followed by
# a fresh private suffix.  The step-t append then adds the new sequence's
# first decoded token.

@dataclasses.dataclass
class Join:
    step: int
    row: int
    shared: List[int]                  # base segment indices kept from the row's path
    suffix: Segment                    # the new private part of the prompt


@dataclasses.dataclass
class DecodeTrace:
    base: Workload
    steps: int
    tokens: np.ndarray                 # int32 [T, b]
    q: np.ndarray                      # float16 [T, b, h, d]
    k: List[np.ndarray]                # per layer: float16 [T, b, h, d]
    v: List[np.ndarray]
    joins: List[Join]                  # in step order

    def joins_at(self, t: int) -> List[Join]:
        return [j for j in self.joins if j.step == t]

    def prompt_tokens(self, j: Join) -> np.ndarray:
        return np.concatenate([self.base.segments[s].tokens for s in j.shared] + [j.suffix.tokens])

    def workload_at(self, t: int) -> Workload:
        """The batch that step t's attention sees: every row's live sequence
        after step t's joins and appends, with the queries of step t."""
        w = self.base
        if not 0 <= t < self.steps:
            raise ValueError(f"step {t} outside [0, {self.steps})")
        segs = list(w.segments)
        paths = [list(p) for p in w.seq_paths]
        start = [0] * w.b
        for j in self.joins:
            if j.step > t:
                break
            segs.append(j.suffix)
            paths[j.row] = list(j.shared) + [len(segs) - 1]
            start[j.row] = j.step
        for r in range(w.b):
            s = start[r]
            segs.append(Segment(tokens=self.tokens[s:t + 1, r],
                                k=[self.k[l][s:t + 1, r] for l in range(w.layers)],
                                v=[self.v[l][s:t + 1, r] for l in range(w.layers)]))
            paths[r].append(len(segs) - 1)
        return Workload(name=f"{w.name}@step{t}", h=w.h, d=w.d, c=w.c, segments=segs,
                        seq_paths=paths, q=self.q[t], layers=w.layers)


def decode_trace(w: Workload, steps: int, seed: int, churn_every: int = 0,
                 suffix=None, unique_starts: bool = False) -> DecodeTrace:
    """Draw a decode trace of ``steps`` iterations over the batch of ``w``.

    Every ``churn_every`` steps (0 = never) one row, drawn uniformly, gets a
    new sequence whose private suffix length is uniform in ``suffix``
    (inclusive; default [c/2, 4c]).  Draw order, from one PCG64 generator
    seeded with ``seed``: tokens [T, b]; per join (in step order) its row,
    suffix length and suffix tokens; Q [T, b, h, d]; then for each layer:
    K [T, b, h, d], V [T, b, h, d], and every join's suffix K then V.
    ``unique_starts``: every join's suffix starts with a token id no segment
    or other join starts with (ids from VOCAB + 2^20 on; use with a base
    workload from ``unique_segment_starts``), so that a join shares exactly
    its shared segments however finely the tree matches tokens."""
    if steps < 1:
        raise ValueError("steps must be >= 1")
    rng = np.random.Generator(np.random.PCG64(seed))
    b, h, d, c = w.b, w.h, w.d, w.c
    lo, hi = suffix if suffix is not None else (max(1, c // 2), 4 * c)
    tokens = rng.integers(0, VOCAB, size=(steps, b), dtype=np.int64).astype(np.int32)
    joins: List[Join] = []
    if churn_every > 0:
        for t in range(churn_every, steps, churn_every):
            row = int(rng.integers(0, b))
            n = int(rng.integers(lo, hi + 1))
            toks = rng.integers(0, VOCAB, size=n, dtype=np.int64).astype(np.int32)
            if unique_starts:
                toks[0] = VOCAB + (1 << 20) + len(joins)
            joins.append(Join(step=t, row=row, shared=list(w.seq_paths[row][:-1]),
                              suffix=Segment(tokens=toks, k=[], v=[])))
    q = _normal_f16(rng, (steps, b, h, d))
    ks, vs = [], []
    for _ in range(w.layers):
        ks.append(_normal_f16(rng, (steps, b, h, d)))
        vs.append(_normal_f16(rng, (steps, b, h, d)))
        for j in joins:
            j.suffix.k.append(_normal_f16(rng, (len(j.suffix), h, d)))
            j.suffix.v.append(_normal_f16(rng, (len(j.suffix), h, d)))
    return DecodeTrace(base=w, steps=steps, tokens=tokens, q=q, k=ks, v=vs, joins=joins)


# ---- prefill batches ------------------------------------------------------------
#
# A prefill batch: sequences arrive whose prompts begin with a prefix that the
# tree already stores (held by a resident sequence that is not part of the
# batch), so only their new tokens need attention (ChunkAttention page,
# Knowl 1 arrival: matched prefix chunks are shared, the newly computed suffix
# tokens get chunks of their own).  Every new token at position p attends to
# the sequence's tokens 0..p.

@dataclasses.dataclass
class PrefillBatch:
    w: Workload
    residents: List[int]              # segments stored (each as a sequence of its own) before the batch
    seqs: List[int]                   # batch sequences (indices into w.seq_paths)
    q_from: List[int]                 # first new position of each batch sequence
    q: np.ndarray                     # float16 [R, h, d], rows in (sequence, position) order

    @property
    def n_rows(self) -> int:
        return int(self.q.shape[0])


def prefill_batch(seed: int, b: int, prefix: int, new, h: int = 2, d: int = 64, c: int = 16,
                  layers: int = 1, with_kv: bool = True, match: str = "chunks") -> PrefillBatch:
    """b sequences = one shared prefix of ``prefix`` tokens + ``new`` tokens
    each (a count or b counts).  The prefix is stored beforehand; its full
    chunks are matched, so every sequence's new rows start at the prefix
    length rounded down to a whole chunk (a partial last prefix chunk is
    written again by each sequence, as whole-chunk matching dictates).
    With ``match="tokens"`` (a token-granular tree) the whole prefix is
    matched, the new rows start at the prefix length, and the workload goes
    through ``unique_segment_starts``.
    Draw order (PCG64(seed)): the workload as ``one_prefix`` draws it
    (tokens, a decode Q that is not used, K/V), then the prefill Q [R, h, d]."""
    newl = [int(new)] * b if np.isscalar(new) else [int(x) for x in new]
    w = one_prefix(seed, b, prefix, newl, h=h, d=d, c=c, layers=layers, with_kv=with_kv)
    if match == "tokens":
        w = unique_segment_starts(w)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    a = prefix if match == "tokens" else (prefix // c) * c
    q_from = [a] * b
    R = sum(w.seq_len(u) - a for u in range(b))
    q = _normal_f16(rng, (R, h, d))
    return PrefillBatch(w=w, residents=[0] if prefix > 0 else [], seqs=list(range(b)),
                        q_from=q_from, q=q)


def prefill_unshared(pb: PrefillBatch) -> PrefillBatch:
    """The same rows, K/V and Q with nothing shared: every sequence holds its
    own copy of the stored prefix under distinct token ids (``unshare``), all
    copies stored before the batch."""
    w = unshare(pb.w)
    residents = [w.seq_paths[u][0] for u in pb.seqs] if pb.residents else []
    return PrefillBatch(w=w, residents=residents, seqs=pb.seqs, q_from=pb.q_from, q=pb.q)
