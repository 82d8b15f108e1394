"""The prefix tree under token-granular matching (PKVT_MATCH_TOKENS),
through the C ABI on the CPU: the hand-worked fixture, random operations
against the token-granular reference model (bit-exact sharing maps, fills,
refcounts), the slots and K/V moves of node splits replayed on an emulated
pool, and rollback when the pool runs out."""
import json
import os

import numpy as np
import pytest

from oracle import sharing as S
from prefix_shared_kv_tree_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(B.LIB_PATH):
        from prefix_shared_kv_tree_amd import build
        build.build()
    return B.load()


class TokenTree:
    def __init__(self, c=4, n=4096, h=2, d=64):
        self.c = c
        self.t = 0
        self.t = B.pkvt_tree_create(h, d, c, n, match="tokens")

    def __del__(self):
        if self.t:
            B.pkvt_tree_destroy(self.t)

    def paths(self, ids):
        return [list(B.pkvt_tree_chunk_path(self.t, int(i))) for i in ids]

    def fills(self, ids):
        return [[B.pkvt_tree_chunk_fill(self.t, int(x)) for x in p] for p in self.paths(ids)]


def test_create_rejects_unknown_match_mode():
    with pytest.raises(B.PkvtError):
        B.pkvt_tree_create(2, 64, 4, 16, match="bytes")


def test_matches_hand_worked_fixture():
    with open(os.path.join(GOLDEN, "token_sharing_c4.json")) as f:
        fx = json.load(f)
    box = TokenTree(c=fx["c"])
    ids = []
    for op in fx["ops"]:
        if op[0] == "insert":
            i, _ = B.pkvt_tree_build(box.t, [op[1]])
            ids.append(int(i[0]))
        elif op[0] == "append":
            B.pkvt_tree_append(box.t, [ids[op[1]]], [op[2]])
        elif op[0] == "remove":
            B.pkvt_tree_remove(box.t, ids[op[1]])
        else:
            exp = op[1]
            live = [ids[k] for k in exp["live"]]
            paths = box.paths(live)
            assert [list(x) for x in S.canonicalize(paths)] == exp["labels"]
            assert box.fills(live) == [[len(n) for n in p] for p in exp["tokens"]]
            assert [[B.pkvt_tree_chunk_refcount(box.t, int(x)) for x in p] for p in paths] == \
                exp["refcounts"]
            assert B.pkvt_tree_stats(box.t)["used_chunks"] == exp["used"]


@pytest.mark.parametrize("seed", range(15))
def test_random_ops_match_reference_model(seed):
    rng = np.random.default_rng(300 + seed)
    c = int(rng.integers(2, 6))
    box = TokenTree(c=c, n=100000)
    model = S.TokenSharingModel(c)
    tree_id = {}
    toks = {}
    for step in range(250):
        r = rng.random()
        live = model.live()
        if r < 0.3 or not live:
            prompts = []
            for _ in range(int(rng.integers(1, 4))):
                base = []
                pool = [toks[m] for m in live] + prompts
                if pool and rng.random() < 0.8:
                    src = pool[int(rng.integers(0, len(pool)))]
                    base = src[:int(rng.integers(0, len(src) + 1))]
                t = base + [int(x) for x in rng.integers(0, 2, size=int(rng.integers(0, 10)))]
                prompts.append(t or [1])
            ids, _ = B.pkvt_tree_build(box.t, prompts)
            for t, i in zip(prompts, ids):
                mid = model.insert(t)
                tree_id[mid] = int(i)
                toks[mid] = list(t)
        elif r < 0.85:
            k = int(rng.integers(1, 4))
            mids = [int(x) for x in rng.choice(live, size=k)]
            tk = [int(x) for x in rng.integers(0, 2, size=k)]
            for m, x in zip(mids, tk):
                model.append(m, x)
                toks[m].append(x)
            B.pkvt_tree_append(box.t, [tree_id[m] for m in mids], tk)
        else:
            m = int(rng.choice(live))
            model.remove(m)
            B.pkvt_tree_remove(box.t, tree_id.pop(m))
            del toks[m]
        live = model.live()
        tids = [tree_id[m] for m in live]
        tpaths = box.paths(tids)
        assert [list(x) for x in S.canonicalize(tpaths)] == \
               [list(x) for x in S.canonicalize(model.paths())], step
        assert box.fills(tids) == [[len(n) for n in model.node_tokens(m)] for m in live]
        rc = model.refcounts()
        for p_t, p_m in zip(tpaths, model.paths()):
            assert [B.pkvt_tree_chunk_refcount(box.t, int(x)) for x in p_t] == [rc[n] for n in p_m]
        for m in live:
            assert B.pkvt_tree_seq_len(box.t, tree_id[m]) == len(toks[m])
        assert B.pkvt_tree_stats(box.t)["used_chunks"] == model.used_chunks()
    for m in list(model.live()):
        B.pkvt_tree_remove(box.t, tree_id[m])
    st = B.pkvt_tree_stats(box.t)
    assert st["used_chunks"] == 0 and st["live_seqs"] == 0


@pytest.mark.parametrize("seed", range(20))
def test_slots_and_moves_place_every_token(seed):
    """Replay builds, appends and removals on an emulated pool (slot -> the
    token's whole prefix, which is what its K/V depend on): write the new
    tokens at their slots and apply each build's moves; afterwards every live
    sequence's path must read its own prefixes back, position by position."""
    rng = np.random.default_rng(900 + seed)
    c = int(rng.integers(2, 6))
    box = TokenTree(c=c, n=100000)
    pool = {}
    toks = {}
    for step in range(120):
        r = rng.random()
        live = list(toks)
        if r < 0.4 or not live:
            prompts = []
            for _ in range(int(rng.integers(1, 5))):
                base = []
                src_pool = [toks[i] for i in live] + prompts
                if src_pool and rng.random() < 0.85:
                    src = src_pool[int(rng.integers(0, len(src_pool)))]
                    base = src[:int(rng.integers(0, len(src) + 1))]
                t = base + [int(x) for x in rng.integers(0, 3, size=int(rng.integers(0, 9)))]
                prompts.append(t or [2])
            ids, slots = B.pkvt_tree_build(box.t, prompts)
            src, dst = B.pkvt_tree_moves(box.t)
            assert not set(src.tolist()) & set(dst.tolist())
            assert all(int(s) in pool for s in src)              # sources hold stored tokens
            off = 0
            new_slots = set()
            for t in prompts:
                for p in range(len(t)):
                    s = int(slots[off + p])
                    if s >= 0:
                        new_slots.add(s)
                off += len(t)
            assert not new_slots & set(src.tolist()) and not new_slots & set(dst.tolist())
            moved = {int(d): pool[int(s)] for s, d in zip(src, dst)}
            pool.update(moved)
            off = 0
            for t, i in zip(prompts, ids):
                for p in range(len(t)):
                    s = int(slots[off + p])
                    if s >= 0:
                        pool[s] = tuple(t[:p + 1])
                off += len(t)
                toks[int(i)] = list(t)
        elif r < 0.85:
            k = int(rng.integers(1, 4))
            who = [int(x) for x in rng.choice(live, size=k)]
            tk = [int(x) for x in rng.integers(0, 3, size=k)]
            slots = B.pkvt_tree_append(box.t, who, tk)
            for i, x, s in zip(who, tk, slots):
                toks[i].append(x)
                pool[int(s)] = tuple(toks[i])
        else:
            i = int(rng.choice(live))
            B.pkvt_tree_remove(box.t, i)
            del toks[i]
        for i, t in toks.items():
            p = 0
            for x in B.pkvt_tree_chunk_path(box.t, i):
                for k in range(B.pkvt_tree_chunk_fill(box.t, int(x))):
                    assert pool[int(x) * c + k] == tuple(t[:p + 1]), (step, i, p)
                    p += 1
            assert p == len(t)


def test_whole_chunk_matching_never_moves():
    t = B.pkvt_tree_create(2, 64, 4, 64)
    try:
        B.pkvt_tree_build(t, [[1, 2, 3, 4, 5, 6], [1, 2, 3, 4, 5, 7]])
        src, dst = B.pkvt_tree_moves(t)
        assert src.size == 0 and dst.size == 0
    finally:
        B.pkvt_tree_destroy(t)


def test_split_moves_listed_and_replaced_by_next_build():
    box = TokenTree(c=4)
    B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5, 6, 7]])          # chunks [1 2 3 4] [5 6 7]
    assert B.pkvt_tree_moves(box.t)[0].size == 0
    ids, slots = B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5, 9]])
    src, dst = B.pkvt_tree_moves(box.t)
    path0 = box.paths([0])[0]
    # [5 6 7] kept [5]; 6 and 7 moved to slots 0 and 1 of the new chunk
    assert len(path0) == 3 and box.fills([0]) == [[4, 1, 2]]
    assert src.tolist() == [path0[1] * 4 + 1, path0[1] * 4 + 2]
    assert dst.tolist() == [path0[2] * 4 + 0, path0[2] * 4 + 1]
    assert slots.tolist()[:5] == [-1] * 5 and slots[5] >= 0
    B.pkvt_tree_build(box.t, [[8]])
    assert B.pkvt_tree_moves(box.t)[0].size == 0


def test_two_splits_of_one_node_in_one_call_compose():
    """A node split twice in one call: each moved token appears once, from
    its original slot to its final one."""
    box = TokenTree(c=8)
    B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5, 6, 7, 8]])
    base = box.paths([0])[0][0] * 8
    B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5, 6, 0], [1, 2, 0]])
    src, dst = B.pkvt_tree_moves(box.t)
    assert sorted(src.tolist()) == [base + k for k in range(2, 8)]
    p0 = box.paths([0])[0]
    assert box.fills([0]) == [[2, 4, 2]]
    final = {base + 2 + k: p0[1] * 8 + k for k in range(4)}
    final.update({base + 6 + k: p0[2] * 8 + k for k in range(2)})
    assert dict(zip(src.tolist(), dst.tolist())) == final


def _state(box, ids):
    return (B.pkvt_tree_stats(box.t), box.paths(ids), box.fills(ids),
            [B.pkvt_tree_seq_len(box.t, i) for i in ids])


def test_pool_exhaustion_with_a_split_rolls_back():
    box = TokenTree(c=4, n=4)
    ids, _ = B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5, 6, 7]])      # 2 chunks
    ids = [int(i) for i in ids]
    before = _state(box, ids)
    with pytest.raises(B.PkvtError) as e:
        # splits [5 6 7] (1 chunk), then needs 2 more for [9 9 9 9 9]: 3 > 2 free
        B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5, 9, 9, 9, 9, 9]])
    assert e.value.status == "NO_CHUNKS"
    assert _state(box, ids) == before
    assert B.pkvt_tree_moves(box.t)[0].size == 0
    ids2, _ = B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5, 9]])        # fits: split + 1 chunk
    assert B.pkvt_tree_stats(box.t)["used_chunks"] == 4


def _plan_and_check(box, order, h, **kw):
    from tests import planview
    mb, wb = B.pkvt_plan(box.t, order, **kw)
    blob = B.pkvt_plan_blob(box.t)
    plan = planview.parse(blob)
    paths = {int(i): [int(x) for x in B.pkvt_tree_chunk_path(box.t, int(i))] for i in order}
    lens = {int(i): B.pkvt_tree_seq_len(box.t, int(i)) for i in order}
    fills = {x: B.pkvt_tree_chunk_fill(box.t, x) for p in paths.values() for x in p}
    planview.check_plan(plan, order, paths, lens, box.c, min_share=kw.get("min_share") or 2,
                        heads=h, unit_rows=kw.get("unit_rows") or 17, fills=fills)
    return plan


@pytest.mark.parametrize("seed", range(25))
def test_plan_invariants_with_partial_nodes(seed):
    """Plans over token-granular trees (partial chunks inside paths, shared
    and private): every (row, chunk) read once, items hold full chunks but
    the last, key counts and key bases follow the fills."""
    rng = np.random.default_rng(1200 + seed)
    c = int(rng.choice([4, 5, 8]))
    h = int(rng.integers(1, 3))
    box = TokenTree(c=c, n=20000, h=h)
    prompts = []
    for _ in range(int(rng.integers(2, 40))):
        base = []
        if prompts and rng.random() < 0.85:
            src = prompts[int(rng.integers(0, len(prompts)))]
            base = src[:int(rng.integers(0, len(src) + 1))]
        prompts.append(base + [int(x) for x in rng.integers(0, 3, size=int(rng.integers(1 if not base else 0, 25)))]
                       or [1])
    ids = [int(i) for i in B.pkvt_tree_build(box.t, prompts)[0]]
    for _ in range(int(rng.integers(0, 30))):                # decode appends grow some leaves
        who = [int(x) for x in rng.choice(ids, size=3)]
        B.pkvt_tree_append(box.t, who, [int(x) for x in rng.integers(0, 3, size=3)])
    for kw in [dict(), dict(phase1_chunks=1, phase2_chunks=1), dict(phase2_chunks=2, unit_rows=17),
               dict(min_share=3), dict(workgroups=3)]:
        order = [int(x) for x in rng.permutation(ids)]
        _plan_and_check(box, order, h, **kw)
    # prefill of every sequence's last few positions (and of whole sequences)
    from tests import planview
    paths = {i: [int(x) for x in B.pkvt_tree_chunk_path(box.t, i)] for i in ids}
    lens = {i: B.pkvt_tree_seq_len(box.t, i) for i in ids}
    fills = {x: B.pkvt_tree_chunk_fill(box.t, x) for p in paths.values() for x in p}
    for q_from in ([0] * len(ids), [max(0, lens[i] - int(rng.integers(1, 9))) for i in ids]):
        B.pkvt_prefill_plan(box.t, ids, q_from)
        plan = planview.parse(B.pkvt_prefill_blob(box.t))
        planview.check_prefill_plan(plan, ids, q_from, paths, lens, c, h, fills=fills)


def test_plan_wide_shared_partial_prefix():
    """40 sequences sharing a 70-token prompt (c = 16: 4 full chunks and a
    6-token chunk, all shared) form workgroup units whose key count ends
    inside the partial chunk."""
    rng = np.random.default_rng(5)
    base = [int(x) for x in rng.integers(0, 1000, size=70)]
    prompts = [base + [2000 + u] + [int(x) for x in rng.integers(0, 1000, size=int(rng.integers(1, 40)))]
               for u in range(40)]
    box = TokenTree(c=16, n=4096, h=2)
    ids = [int(i) for i in B.pkvt_tree_build(box.t, prompts)[0]]
    plan = _plan_and_check(box, ids, 2)
    assert len(plan["units"]) > 0
    assert sorted({int(u[0]) for u in plan["units"]}) == [70]
    # prefill of the private tokens: rows read the shared 70 tokens (a unit
    # ending inside chunk 4) and then their own chunks, whose keys start at 70
    from tests import planview
    q_from = [71] * len(ids)
    B.pkvt_prefill_plan(box.t, ids, q_from)
    pplan = planview.parse(B.pkvt_prefill_blob(box.t))
    paths = {i: [int(x) for x in B.pkvt_tree_chunk_path(box.t, i)] for i in ids}
    lens = {i: B.pkvt_tree_seq_len(box.t, i) for i in ids}
    fills = {x: B.pkvt_tree_chunk_fill(box.t, x) for p in paths.values() for x in p}
    assert sorted(fills[p[4]] for p in paths.values())[0] == 6
    planview.check_prefill_plan(pplan, ids, q_from, paths, lens, 16, 2, fills=fills)
    assert 70 in {int(u[7]) for u in pplan["units"]}


def test_new_entry_points_reject_bad_arguments(lib):
    import ctypes as C
    t = B.pkvt_tree_create(2, 64, 4, 8, match="tokens")
    try:
        n = C.c_int64()
        assert lib.pkvt_tree_moves(t, None, None, 0, None) == -1          # NULL count
        assert lib.pkvt_tree_moves(None, None, None, 0, C.byref(n)) == -1
        f = C.c_int32()
        assert lib.pkvt_tree_chunk_fill(t, 8, C.byref(f)) == -1           # chunk id out of range
        assert lib.pkvt_tree_chunk_fill(t, 0, None) == -1
        B.pkvt_tree_build(t, [[1, 2, 3, 4, 5]])
        B.pkvt_tree_build(t, [[1, 2, 9]])                                 # splits [1 2 3 4]
        assert lib.pkvt_tree_moves(t, None, None, 0, C.byref(n)) == -6    # BUFFER_TOO_SMALL
        assert n.value == 2
        src = (C.c_int64 * 2)()
        assert lib.pkvt_tree_moves(t, src, None, 2, C.byref(n)) == -1     # NULL dst
    finally:
        B.pkvt_tree_destroy(t)
    # kv_move: argument checks happen before any device work
    t = B.pkvt_tree_create(2, 64, 16, 8, match="tokens")
    try:
        assert lib.pkvt_kv_move(t, None, None, None, None, -1, None) == -1
        assert lib.pkvt_kv_move(t, None, None, None, None, 0, None) == 0
        assert lib.pkvt_kv_move(t, None, None, None, None, 3, None) == -1
    finally:
        B.pkvt_tree_destroy(t)
    odd = B.pkvt_tree_create(2, 32, 4, 8)                                 # head_dim 32: no kernels
    try:
        assert lib.pkvt_kv_move(odd, None, None, None, None, 1, None) == -5
    finally:
        B.pkvt_tree_destroy(odd)
    out = C.c_void_p()
    assert lib.pkvt_tree_create_ex(2, 64, 4, 8, 7, C.byref(out)) == -1 and not out.value
