"""Host side of the decode loop, on the CPU: the seeded decode traces, and
the tree and plans that HostDecoder keeps while sequences append, leave and
arrive (ChunkAttention page, Knowl 1: arrival, decoding iteration and
departure; Knowl 5: re-planning only after structural changes)."""
import numpy as np
import pytest

from oracle import sharing as S
from prefix_shared_kv_tree_amd import binding as B
from prefix_shared_kv_tree_amd import workloads as W
from prefix_shared_kv_tree_amd.harness import HostDecoder, loop_pool_chunks

from . import planview as PV


def test_trace_is_seeded_and_consistent():
    w = W.make_config("tiny", layers=2)
    a = W.decode_trace(w, 30, seed=11, churn_every=7)
    b = W.decode_trace(w, 30, seed=11, churn_every=7)
    assert np.array_equal(a.tokens, b.tokens) and np.array_equal(a.q, b.q)
    assert all(np.array_equal(x, y) for x, y in zip(a.k + a.v, b.k + b.v))
    assert [(j.step, j.row, len(j.suffix)) for j in a.joins] == \
        [(j.step, j.row, len(j.suffix)) for j in b.joins]
    assert [j.step for j in a.joins] == [7, 14, 21, 28]
    for t in (0, 6, 7, 29):
        wt = a.workload_at(t)
        assert np.array_equal(wt.q, a.q[t])
        for r in range(w.b):
            js = [j for j in a.joins if j.row == r and j.step <= t]
            if js:
                j = js[-1]
                assert wt.seq_len(r) == 64 + len(j.suffix) + (t + 1 - j.step)
                assert np.array_equal(wt.seq_tokens(r)[:64], w.segments[0].tokens)
                assert np.array_equal(wt.seq_tokens(r)[64:64 + len(j.suffix)], j.suffix.tokens)
            else:
                assert wt.seq_len(r) == w.seq_len(r) + t + 1
                assert np.array_equal(wt.seq_tokens(r)[:w.seq_len(r)], w.seq_tokens(r))
            # the decoded tokens of the live sequence, newest last, with their K/V
            assert wt.seq_tokens(r)[-1] == a.tokens[t, r]
            last = wt.segments[wt.seq_paths[r][-1]]
            assert np.array_equal(last.k[1][-1], a.k[1][t, r])
    with pytest.raises(ValueError):
        a.workload_at(30)


def _check_tree(hd, wt):
    """The live rows' chunk paths follow the sharing definition for their
    current token sequences; refcounts count rows; nothing else is held."""
    tree = hd.tree
    paths = [B.pkvt_tree_chunk_path(tree, int(s)) for s in hd.rows]
    toks = wt.all_seq_tokens()
    for r, s in enumerate(hd.rows):
        assert B.pkvt_tree_seq_len(tree, int(s)) == len(toks[r])
    labels = S.chunk_labels(toks, wt.c)
    assert [list(x) for x in S.canonicalize(paths)] == [list(x) for x in labels]
    cov = S.coverage(labels)
    phys = {}
    for p, labs in zip(paths, labels):
        for x, l in zip(p, labs):
            phys[int(l)] = int(x)
    for lab, users in cov.items():
        assert B.pkvt_tree_chunk_refcount(tree, phys[lab]) == len(users)
    st = B.pkvt_tree_stats(tree)
    assert st["used_chunks"] == len(cov)
    assert st["live_seqs"] == wt.b
    return paths


@pytest.mark.parametrize("name,steps,churn,check_every", [
    ("tiny", 60, 5, 1),
    ("c4", 70, 9, 23),
    ("c3", 70, 8, 23),
    ("c3", 90, 45, 1),
])
def test_host_decoder_follows_trace(name, steps, churn, check_every):
    w = W.make_config(name, with_kv=False)
    tr = W.decode_trace(w, steps, seed=77, churn_every=churn,
                        suffix=(256, 1024) if name == "c3" else None)
    t = B.pkvt_tree_create(w.h, w.d, w.c, loop_pool_chunks(tr))
    try:
        ids, _ = B.pkvt_tree_build(t, w.all_seq_tokens())
        hd = HostDecoder(t, tr, ids)
        hd.plan()
        full0 = hd.count["plan_full"]
        structural_steps = 0
        for step in range(steps):
            joined = hd.joins(step)
            for j, slots, _ in joined:
                # the kept shared prefix is already stored: only the tail of a
                # partially filled chunk and the suffix need writing
                n_pre = sum(len(w.segments[s]) for s in j.shared)
                assert np.all(slots[:n_pre - n_pre % w.c] == -1)
                assert np.all(slots[n_pre:] >= 0)
            slots = hd.append(step)
            # the new token goes right after the sequence's last one
            for r, s in enumerate(hd.rows):
                p = B.pkvt_tree_chunk_path(t, int(s))
                n = B.pkvt_tree_seq_len(t, int(s))
                assert slots[r] == p[-1] * w.c + (n - 1) % w.c
            structural_steps += bool(joined) or bool(np.any(slots % w.c == 0))
            hd.plan()
            if step % check_every == 0 or step == steps - 1:
                wt = tr.workload_at(step)
                paths = _check_tree(hd, wt)
                plan = PV.parse(B.pkvt_plan_blob(t))
                PV.check_plan(plan, hd.rows, {int(s): p for s, p in zip(hd.rows, paths)},
                              {int(s): wt.seq_len(r) for r, s in enumerate(hd.rows)}, w.c,
                              heads=w.h)
        assert hd.count["plan_full"] + hd.count["plan_patch"] - full0 == structural_steps
        assert hd.count["plan_refresh"] == steps - structural_steps
        # appends that open leaf chunks are patched in; full rebuilds follow
        # arrivals (or a row whose reserved room ran out)
        if name != "tiny":
            assert hd.count["plan_patch"] > 0
            assert hd.count["plan_full"] - full0 <= len(tr.joins) + steps // w.c + 1
        assert hd.count["join"] == len(tr.joins)
        # every row leaves: the pool is whole again
        for s in hd.rows:
            B.pkvt_tree_remove(t, int(s))
        st = B.pkvt_tree_stats(t)
        assert st["used_chunks"] == 0 and st["free_chunks"] == st["capacity"]
    finally:
        B.pkvt_tree_destroy(t)


@pytest.mark.parametrize("seed,c", [(5, 16), (6, 32), (7, 4)])
def test_host_decoder_token_matching(seed, c):
    """HostDecoder on a token-granular tree: a shared prompt that ends inside
    a chunk, joins whose prompts split nodes of live sequences.  Replays the
    slots and each join's K/V moves on an emulated pool (slot -> the token's
    whole prefix, which is what its K/V depend on) and checks every live
    sequence's path against it, plus the plan invariants with partial
    chunks."""
    rng = np.random.default_rng(seed)
    b = 10
    prefix = 3 * c + int(rng.integers(1, c))
    w = W.unique_segment_starts(W.one_prefix(seed, b, prefix, [int(x) for x in rng.integers(1, 3 * c, b)],
                                             h=1, d=64, c=c, with_kv=False))
    tr = W.decode_trace(w, 3 * c + 7, seed=seed, churn_every=4, suffix=(1, 2 * c), unique_starts=True)
    t = B.pkvt_tree_create(w.h, w.d, w.c, loop_pool_chunks(tr), match="tokens")
    try:
        # the batch arrives one prompt per call: the second splits the first's
        # node at the prompt's end, whose tail K/V moves
        prompts = [list(int(x) for x in p) for p in w.all_seq_tokens()]
        pool = {}
        moved = 0
        ids = []
        for p in prompts:
            i, sl = B.pkvt_tree_build(t, [p])
            src, dst = B.pkvt_tree_moves(t)
            pool.update({int(d): pool[int(s)] for s, d in zip(src, dst)})
            moved += src.size
            for k in range(len(p)):
                if sl[k] >= 0:
                    pool[int(sl[k])] = tuple(p[:k + 1])
            ids.append(int(i[0]))
        assert moved > 0
        seqs = {i: list(p) for i, p in zip(ids, prompts)}
        hd = HostDecoder(t, tr, np.array(ids, np.int32))
        hd.plan()
        for step in range(tr.steps):
            old_rows = [int(x) for x in hd.rows]
            for j, sl, (src, dst) in hd.joins(step):
                assert not set(src.tolist()) & set(dst.tolist())
                pool.update({int(d): pool[int(s)] for s, d in zip(src, dst)})
                moved += src.size
                p = [int(x) for x in tr.prompt_tokens(j)]
                for k in range(len(p)):
                    if sl[k] >= 0:
                        pool[int(sl[k])] = tuple(p[:k + 1])
                del seqs[old_rows[j.row]]
                seqs[int(hd.rows[j.row])] = p
            sl = hd.append(step)
            for r, s in enumerate(hd.rows):
                seqs[int(s)].append(int(tr.tokens[step, r]))
                pool[int(sl[r])] = tuple(seqs[int(s)])
            hd.plan()
            for s, toks in seqs.items():
                pos = 0
                for x in B.pkvt_tree_chunk_path(t, s):
                    for k in range(B.pkvt_tree_chunk_fill(t, int(x))):
                        assert pool[int(x) * c + k] == tuple(toks[:pos + 1]), (step, s, pos)
                        pos += 1
                assert pos == len(toks)
            plan = PV.parse(B.pkvt_plan_blob(t))
            paths = {int(s): [int(x) for x in B.pkvt_tree_chunk_path(t, int(s))] for s in hd.rows}
            fills = {x: B.pkvt_tree_chunk_fill(t, x) for p in paths.values() for x in p}
            PV.check_plan(plan, hd.rows, paths, {int(s): len(seqs[int(s)]) for s in hd.rows}, c,
                          heads=w.h, fills=fills)
    finally:
        B.pkvt_tree_destroy(t)
