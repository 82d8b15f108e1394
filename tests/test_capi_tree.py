"""Host side of libpkvt through its C ABI, on the CPU: exported symbols, the
prefix tree against the sharing-map oracle (bit-exact), dynamic operations
against the reference model, error paths, and the plan's invariants."""
import json
import os
import re

import numpy as np
import pytest

from oracle import sharing as S
from prefix_shared_kv_tree_amd import binding as B
from prefix_shared_kv_tree_amd import workloads as W
from tests import planview

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(B.LIB_PATH):
        from prefix_shared_kv_tree_amd import build
        build.build()
    return B.load()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "pkvt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkvt_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    declared = _header_functions()
    assert len(declared) >= 16
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(B.exported_symbols()) == declared


class TreeBox:
    def __init__(self, h=2, d=64, c=4, n=4096):
        self.h, self.d, self.c = h, d, c
        self.t = 0
        self.t = B.pkvt_tree_create(h, d, c, n)

    def __del__(self):
        if self.t:
            B.pkvt_tree_destroy(self.t)

    def paths(self, ids):
        return [B.pkvt_tree_chunk_path(self.t, int(i)) for i in ids]


def _check_build_against_definition(box, seqs):
    ids, slots = B.pkvt_tree_build(box.t, seqs)
    paths = box.paths(ids)
    got = [list(x) for x in S.canonicalize(paths)]
    want = [list(x) for x in S.chunk_labels(seqs, box.c)]
    assert got == want
    # refcount of a chunk = number of sequences through it
    cov = S.coverage(S.chunk_labels(seqs, box.c))
    first_phys = {}
    for p, labs in zip(paths, S.chunk_labels(seqs, box.c)):
        for x, l in zip(p, labs):
            first_phys[int(l)] = int(x)
    for lab, users in cov.items():
        assert B.pkvt_tree_chunk_refcount(box.t, first_phys[lab]) == len(users)
    # slots: -1 exactly for tokens in chunks that existed before the sequence
    pos = 0
    seen = set()
    for u, (p, toks) in enumerate(zip(paths, seqs)):
        for k, x in enumerate(p):
            n = min(box.c, len(toks) - k * box.c)
            sl = slots[pos + k * box.c: pos + k * box.c + n]
            if int(x) in seen:
                assert np.all(sl == -1)
            else:
                assert list(sl) == [int(x) * box.c + j for j in range(n)]
                seen.add(int(x))
        pos += len(toks)
    st = B.pkvt_tree_stats(box.t)
    assert st["used_chunks"] == len(cov)
    assert st["shared_chunks"] == sum(1 for v in cov.values() if len(v) >= 2)
    return ids, paths


@pytest.mark.parametrize("seed", range(30))
def test_build_matches_sharing_definition_random(seed):
    w = W.random_tree(seed, c=4, max_b=8, max_len=50, vocab=2)
    _check_build_against_definition(TreeBox(c=4), w.all_seq_tokens())


@pytest.mark.parametrize("name", ["tiny", "c2", "c3", "c4", "c5"])
def test_build_matches_sharing_definition_configs(name):
    w = W.make_config(name, with_kv=False)
    box = TreeBox(h=w.h, d=w.d, c=w.c, n=4096)
    _check_build_against_definition(box, w.all_seq_tokens())


def test_build_incremental_calls_match_single_call():
    w = W.random_tree(5, c=4, max_b=8, max_len=50, vocab=2)
    seqs = w.all_seq_tokens()
    box = TreeBox(c=4)
    ids = []
    for s in seqs:
        i, _ = B.pkvt_tree_build(box.t, [s])
        ids.append(int(i[0]))
    got = [list(x) for x in S.canonicalize(box.paths(ids))]
    assert got == [list(x) for x in S.chunk_labels(seqs, 4)]


def test_dynamic_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "dynamic_sharing_c4.json")))
    box = TreeBox(c=fx["c"])
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
            assert [[B.pkvt_tree_chunk_refcount(box.t, int(x)) for x in p] for p in paths] == exp["refcounts"]
            assert B.pkvt_tree_stats(box.t)["used_chunks"] == exp["used"]


@pytest.mark.parametrize("seed", range(15))
def test_random_ops_match_reference_model(seed):
    rng = np.random.default_rng(100 + seed)
    c = 4
    box = TreeBox(c=c, n=100000)
    model = S.SharingModel(c)
    tree_id = {}          # model id -> tree id
    toks = {}
    for step in range(250):
        r = rng.random()
        live = model.live()
        if r < 0.3 or not live:
            base = []
            if live and rng.random() < 0.7:
                src = toks[int(rng.choice(live))]
                base = src[:int(rng.integers(0, len(src) + 1))]
            t = base + [int(x) for x in rng.integers(0, 2, size=int(rng.integers(0, 10)))]
            if not t:
                t = [1]
            mid = model.insert(t)
            i, _ = B.pkvt_tree_build(box.t, [t])
            tree_id[mid] = int(i[0])
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
        tpaths = box.paths([tree_id[m] for m in live])
        assert [list(x) for x in S.canonicalize(tpaths)] == \
               [list(x) for x in S.canonicalize(model.paths())], step
        rc = model.refcounts()
        for p_t, p_m in zip(tpaths, model.paths()):
            assert [B.pkvt_tree_chunk_refcount(box.t, int(x)) for x in p_t] == [rc[n] for n in p_m]
        for m in live:
            assert B.pkvt_tree_seq_len(box.t, tree_id[m]) == len(toks[m])
        assert B.pkvt_tree_stats(box.t)["used_chunks"] == model.used_chunks()
    for m in list(model.live()):
        B.pkvt_tree_remove(box.t, tree_id[m])
    st = B.pkvt_tree_stats(box.t)
    assert st["used_chunks"] == 0 and st["free_chunks"] == st["capacity"] and st["live_seqs"] == 0


def _snapshot(box, ids):
    return (B.pkvt_tree_stats(box.t), [list(p) for p in box.paths(ids)],
            [B.pkvt_tree_seq_len(box.t, i) for i in ids])


def test_pool_exhaustion_build_rolls_back():
    box = TreeBox(c=4, n=6)
    ids, _ = B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5, 6, 7, 8, 9]])       # 3 chunks
    before = _snapshot(box, ids)
    with pytest.raises(B.PkvtError) as e:
        # the first prompt fits (shares 2, adds 2), the second does not
        B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5, 6, 7, 8, 7, 7, 7, 7, 1], [9, 9, 9, 9, 9]])
    assert e.value.status == "NO_CHUNKS"
    assert _snapshot(box, ids) == before
    # and the pool still works afterwards
    ids2, _ = B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 0]])
    assert B.pkvt_tree_stats(box.t)["used_chunks"] == 4


def test_pool_exhaustion_append_rolls_back():
    box = TreeBox(c=2, n=3)
    ids, _ = B.pkvt_tree_build(box.t, [[1, 2], [1, 2, 3]])               # chunks: [1,2] shared, [3]
    before = _snapshot(box, ids)
    with pytest.raises(B.PkvtError) as e:
        # seq0 needs a new chunk (leaf full+shared): uses the last free one; seq1 fills [3,4]
        # then needs another -> exhausted
        B.pkvt_tree_append(box.t, [ids[0], ids[1], ids[1]], [5, 4, 6])
    assert e.value.status == "NO_CHUNKS"
    assert _snapshot(box, ids) == before


def test_unknown_and_double_remove():
    box = TreeBox(c=4)
    ids, _ = B.pkvt_tree_build(box.t, [[1, 2, 3]])
    B.pkvt_tree_remove(box.t, ids[0])
    for fn in (lambda: B.pkvt_tree_remove(box.t, ids[0]),
               lambda: B.pkvt_tree_append(box.t, [ids[0]], [1]),
               lambda: B.pkvt_tree_seq_len(box.t, 12345),
               lambda: B.pkvt_tree_chunk_path(box.t, 777)):
        with pytest.raises(B.PkvtError) as e:
            fn()
        assert e.value.status == "UNKNOWN_SEQ"


def test_empty_prompt_rejected_and_nothing_inserted():
    box = TreeBox(c=4)
    with pytest.raises(B.PkvtError) as e:
        B.pkvt_tree_build(box.t, [[1, 2], []])
    assert e.value.status == "EMPTY_SEQ"
    assert B.pkvt_tree_stats(box.t)["live_seqs"] == 0
    assert B.pkvt_tree_stats(box.t)["used_chunks"] == 0


@pytest.mark.parametrize("d,c", [(32, 16), (96, 64), (128, 8), (128, 48), (512, 64), (256, 256)])
def test_unsupported_shapes(d, c):
    """Host tree works for any shape; device entry points refuse before
    touching the GPU."""
    box = TreeBox(h=2, d=d, c=c)
    ids, _ = B.pkvt_tree_build(box.t, [[1] * 70, [1] * 80])
    B.pkvt_plan(box.t, ids)
    for fn in (lambda: B.pkvt_pool_bytes(4, d, c, 10),
               lambda: B.pkvt_plan_upload(box.t, 0x1000, 1 << 20),
               lambda: B.pkvt_attn_decode(box.t, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0.1),
               lambda: B.pkvt_kv_scatter(box.t, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1)):
        with pytest.raises(B.PkvtError) as e:
            fn()
        assert e.value.status == "UNSUPPORTED_SHAPE"


@pytest.mark.parametrize("args", [(0, 64, 16, 10), (2, 0, 16, 10), (2, 64, 0, 10),
                                  (2, 64, 5000, 10), (2, 64, 16, 0)])
def test_create_rejects_bad_sizes(args):
    with pytest.raises(B.PkvtError) as e:
        B.pkvt_tree_create(*args)
    assert e.value.status == "INVALID_ARG"


def test_pool_bytes():
    assert B.pkvt_pool_bytes(32, 128, 64, 10) == 10 * 32 * 64 * 128 * 2


def test_plan_errors():
    box = TreeBox(c=4)
    ids, _ = B.pkvt_tree_build(box.t, [[1, 2, 3], [1, 2, 3, 4, 5]])
    for order, status in [([], "INVALID_ARG"), ([ids[0], ids[0]], "INVALID_ARG"),
                          ([ids[0], 99], "UNKNOWN_SEQ")]:
        with pytest.raises(B.PkvtError) as e:
            B.pkvt_plan(box.t, order)
        assert e.value.status == status
    with pytest.raises(B.PkvtError) as e:
        B.pkvt_plan(box.t, list(ids), min_share=1)
    assert e.value.status == "INVALID_ARG"


def test_stale_plan_rejected_on_cpu_calls():
    box = TreeBox(c=4)
    ids, _ = B.pkvt_tree_build(box.t, [[1, 2, 3], [1, 2, 3, 4, 5]])
    B.pkvt_plan(box.t, ids)
    B.pkvt_tree_append(box.t, [ids[0]], [9])
    # upload checks staleness before touching the device
    with pytest.raises(B.PkvtError) as e:
        B.pkvt_plan_upload(box.t, 0x1000, 1 << 20)
    assert e.value.status == "STALE_PLAN"
    with pytest.raises(B.PkvtError) as e:
        B.pkvt_attn_decode(box.t, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0.125)
    assert e.value.status == "STALE_PLAN"


def _plan_and_check(box, order, **kw):
    mb, wb = B.pkvt_plan(box.t, order, **kw)
    blob = B.pkvt_plan_blob(box.t)
    assert mb == 4 * blob.size
    plan = planview.parse(blob)
    assert plan["total"] == blob.size
    live = list(order)
    paths = {int(i): list(B.pkvt_tree_chunk_path(box.t, int(i))) for i in live}
    lens = {int(i): B.pkvt_tree_seq_len(box.t, int(i)) for i in live}
    planview.check_plan(plan, order, paths, lens, box.c, min_share=kw.get("min_share") or 2,
                        heads=box.h, unit_rows=kw.get("unit_rows") or 17)
    assert wb == plan["n_slots"] * box.h * (box.d + 2) * 4
    return plan


@pytest.mark.parametrize("seed", range(30))
def test_plan_invariants_random(seed):
    rng = np.random.default_rng(seed)
    w = W.random_tree(seed, c=4, max_b=9, max_len=70, vocab=2)
    box = TreeBox(c=4)
    ids, _ = B.pkvt_tree_build(box.t, w.all_seq_tokens())
    for trial in range(3):
        k = int(rng.integers(1, len(ids) + 1))
        order = [int(x) for x in rng.permutation(ids)[:k]]
        p1 = int(rng.integers(0, 4))
        p2 = int(rng.integers(0, 4))
        ms = int(rng.choice([0, 2, 3, 100]))
        _plan_and_check(box, order, phase1_chunks=p1, phase2_chunks=p2, min_share=ms)


@pytest.mark.parametrize("seed", range(10))
def test_plan_invariants_wide(seed):
    """Many sequences per shared node: phase-1 row blocks of 17..64 rows
    become workgroup units, longer ones are cut at 64 rows."""
    rng = np.random.default_rng(100 + seed)
    h = int(rng.integers(1, 4))
    w = W.layered_tree(100 + seed, int(rng.integers(20, 161)), int(rng.integers(1, 4)), h=h, c=4)
    box = TreeBox(h=h, c=4, n=8192)
    ids, _ = B.pkvt_tree_build(box.t, w.all_seq_tokens())
    cover = {}
    for i in ids:
        for x in B.pkvt_tree_chunk_path(box.t, int(i)):
            cover[int(x)] = cover.get(int(x), 0) + 1
    for p1, p2, ms in [(0, 0, 0), (1, 1, 0), (3, 2, 5), (0, 0, 17)]:
        plan = _plan_and_check(box, [int(x) for x in rng.permutation(ids)],
                               phase1_chunks=p1, phase2_chunks=p2, min_share=ms)
        wide = any(n >= max(17, ms) for n in cover.values())
        assert (len(plan["units"]) > 0) == wide
    order = [int(x) for x in ids]
    assert len(_plan_and_check(box, order, unit_rows=65)["units"]) == 0
    plan = _plan_and_check(box, order, unit_rows=40)
    assert all(int(u[5]) >= 40 for u in plan["units"])
    with pytest.raises(B.PkvtError):
        B.pkvt_plan(box.t, order, unit_rows=16)


def test_plan_invariants_after_dynamic_ops():
    rng = np.random.default_rng(7)
    box = TreeBox(c=4)
    ids, _ = B.pkvt_tree_build(box.t, [[1] * 9, [1] * 13, [1] * 4 + [2] * 6, [3] * 5])
    live = [int(i) for i in ids]
    for step in range(60):
        if rng.random() < 0.7:
            who = [int(x) for x in rng.choice(live, size=3)]
            B.pkvt_tree_append(box.t, who, [int(x) for x in rng.integers(0, 2, size=3)])
        else:
            i, _ = B.pkvt_tree_build(box.t, [[1] * int(rng.integers(1, 12))])
            live.append(int(i[0]))
        if len(live) > 3 and rng.random() < 0.2:
            B.pkvt_tree_remove(box.t, live.pop(int(rng.integers(0, len(live)))))
        _plan_and_check(box, list(rng.permutation(live)), phase2_chunks=int(rng.integers(0, 3)))


@pytest.mark.parametrize("name", ["tiny", "c2", "c3", "c4", "c5"])
def test_plan_on_configs(name):
    w = W.make_config(name, with_kv=False)
    box = TreeBox(h=w.h, d=w.d, c=w.c, n=4096)
    ids, _ = B.pkvt_tree_build(box.t, w.all_seq_tokens())
    plan = _plan_and_check(box, ids)
    info = B.pkvt_plan_info_get(box.t)
    labs = S.chunk_labels(w.all_seq_tokens(), w.c)
    cov = S.coverage(labs)
    assert info["shared_chunks"] == sum(1 for v in cov.values() if len(v) >= 2)
    assert info["unique_tokens"] == W.unique_tokens(w)
    assert info["logical_tokens"] == W.logical_tokens(w)
    if name == "c5":
        assert info["phase1_items"] == 0 and info["shared_chunks"] == 0
    # plain mode: nothing in phase 1
    _plan_and_check(box, ids, min_share=1 << 20)
    assert B.pkvt_plan_info_get(box.t)["phase1_items"] == 0


def test_plan_refresh_after_length_only_append():
    box = TreeBox(c=4)
    ids, _ = B.pkvt_tree_build(box.t, [[1, 2, 3, 4, 5], [1, 2, 3, 4, 6, 7]])
    B.pkvt_plan(box.t, ids)
    v0 = B.pkvt_plan_info_get(box.t)["structure_version"]
    B.pkvt_tree_append(box.t, [ids[0]], [8])          # fills the private leaf, no new chunk
    B.pkvt_plan(box.t, ids)
    assert B.pkvt_plan_info_get(box.t)["structure_version"] == v0
    blob = planview.parse(B.pkvt_plan_blob(box.t))
    assert sorted(blob["seqlen"].tolist()) == [6, 6]
    B.pkvt_tree_append(box.t, [ids[0]] * 3, [9, 10, 11])   # fills [5,8,9,10], opens [11]
    B.pkvt_plan(box.t, ids)
    assert B.pkvt_plan_info_get(box.t)["structure_version"] != v0


@pytest.mark.parametrize("rows,unit_rows,want_units,want_single_rows", [
    (80, 0, [40, 40], []),           # 64 + 16 would leave a 16-row single-wave task
    (65, 0, [33, 32], []),
    (96, 0, [64, 32], []),           # the 32-row remainder is a unit already
    (130, 0, [44, 43, 43], []),      # not 64 + 64 + a 2-row single-wave task
    (150, 0, [64, 64, 22], []),      # the 22-row remainder is a unit already
    (70, 40, [64], [6]),             # equal blocks of 35 would be below unit_rows
    (64, 0, [64], []),
    (16, 0, [], [16]),
])
def test_phase1_row_blocks(rows, unit_rows, want_units, want_single_rows):
    """How the rows of one shared prefix are cut into workgroup units (17..64
    rows) and single-wave tasks (<= 16 rows)."""
    w = W.one_prefix(9, rows, 8, 0, h=1, d=64, c=4, with_kv=False)
    box = TreeBox(h=1, c=4, n=4096)
    ids, _ = B.pkvt_tree_build(box.t, w.all_seq_tokens())
    plan = _plan_and_check(box, ids, phase1_chunks=2, unit_rows=unit_rows)
    got_units = sorted((int(u[5]) for u in plan["units"]), reverse=True)
    shared = [i for i, ch in enumerate(plan["wave_chunks"]) if len(ch) and
              all(B.pkvt_tree_chunk_refcount(box.t, int(x)) > 1 for x in ch)]
    assert sorted(want_units, reverse=True) == got_units    # one item: 8 tokens = 2 chunks
    assert sorted(int(plan["waves"][i][5]) for i in shared) == sorted(want_single_rows)


@pytest.mark.parametrize("n_s,want_items,floor_items", [(1024, 8, 4), (2048, 8, 7), (4096, 8, 8)])
def test_units_only_plan_fills_the_grid(n_s, want_items, floor_items):
    """A batch whose rows are all shared (32 rows over one prefix, 32 heads,
    d = 128) runs on the units-only kernel, one workgroup per compute unit
    (256 of the default 512), and is cut into about one unit per workgroup --
    8 items x 32 heads -- even where the partial-cost floor alone (items long
    enough that their partials cost at most a quarter of their K/V bytes:
    5 chunks here) would leave the grid partly idle."""
    w = W.one_prefix(21, 32, n_s, 0, h=32, d=128, c=64, with_kv=False)
    box = TreeBox(h=32, d=128, c=64, n=256)
    ids, _ = B.pkvt_tree_build(box.t, w.all_seq_tokens())
    plan = _plan_and_check(box, ids)
    info = B.pkvt_plan_info_get(box.t)
    assert info["kernel"] == 1
    assert info["phase1_items"] == want_items and info["wg_units"] == want_items * 32 == 256
    # the floor: ceil(8 R (d + 2) 4 / (4 c d)) chunks per item, R = 32
    need = -(-8 * 32 * 130 * 4 // (4 * 64 * 128))
    assert need == 5 and -(-(n_s // 64) // max(need, (n_s // 64) // 8)) == floor_items
    assert all(int(u[5]) == 32 for u in plan["units"])
