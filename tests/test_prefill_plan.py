"""Prefill plans on the CPU (no GPU needed): every query row reads exactly
its sequence's keys 0 .. p once, from its own path, in blocks of at most 64
rows; rows of sequences that share stored chunks are batched."""
import numpy as np
import pytest

from prefix_shared_kv_tree_amd import binding as B
from prefix_shared_kv_tree_amd import workloads as W

from . import planview as PV


def _tree(h, d, c, n=20000):
    return B.pkvt_tree_create(h, d, c, n)


def _check(t, ids, q_from, c, h, **kw):
    mb, wb = B.pkvt_prefill_plan(t, ids, q_from, **kw)
    blob = B.pkvt_prefill_blob(t)
    assert mb == 4 * blob.size
    plan = PV.parse(blob)
    paths = {int(s): list(B.pkvt_tree_chunk_path(t, int(s))) for s in ids}
    lens = {int(s): B.pkvt_tree_seq_len(t, int(s)) for s in ids}
    PV.check_prefill_plan(plan, ids, q_from, paths, lens, c, h)
    info = B.pkvt_prefill_info_get(t)
    assert info["b"] == plan["b"] and info["slots"] == plan["n_slots"]
    assert wb == plan["n_slots"] * h * (64 + 2) * 4          # every tree here has d = 64
    return plan, info


@pytest.mark.parametrize("b,prefix,new,c", [(1, 0, 40, 16), (3, 40, [5, 0, 20], 16), (20, 64, 17, 16),
                                            (70, 96, 3, 32), (5, 200, [130, 1, 64, 65, 7], 64)])
def test_prefill_batch_plans(b, prefix, new, c):
    pb = W.prefill_batch(7, b, prefix, new, h=2, d=64, c=c, with_kv=False)
    t = _tree(2, 64, c)
    try:
        if pb.residents:
            B.pkvt_tree_build(t, [pb.w.segments[s].tokens for s in pb.residents])
        ids, slots = B.pkvt_tree_build(t, [pb.w.seq_tokens(u) for u in pb.seqs])
        plan, info = _check(t, ids, pb.q_from, c, 2)
        if prefix >= c and b > 1:
            assert info["shared_chunks"] >= prefix // c
        for ch in (1, 3):
            _check(t, ids, pb.q_from, c, 2, phase1_chunks=ch)
    finally:
        B.pkvt_tree_destroy(t)


def test_shared_prefix_read_once_per_row_block():
    """64 sequences x 8 new tokens over a stored 4-chunk prefix: 512 rows in
    blocks of 32 sequences (256 rows), so each prefix chunk is read by 2 row
    blocks (per head), not 64."""
    pb = W.prefill_batch(3, 64, 64, 8, h=1, d=64, c=16, with_kv=False)
    t = _tree(1, 64, 16)
    try:
        B.pkvt_tree_build(t, [pb.w.segments[s].tokens for s in pb.residents])
        ids, _ = B.pkvt_tree_build(t, [pb.w.seq_tokens(u) for u in pb.seqs])
        plan, _ = _check(t, ids, pb.q_from, 16, 1)
        prefix_chunks = set(int(x) for x in B.pkvt_tree_chunk_path(t, int(ids[0]))[:4])
        readers = [u for u, ch in zip(plan["units"], plan["unit_chunks"])
                   if prefix_chunks & set(int(x) for x in ch)]
        assert len(readers) == 2 and all(int(u[5]) == 256 for u in readers)
    finally:
        B.pkvt_tree_destroy(t)


@pytest.mark.parametrize("seed", range(12))
def test_random_trees_first_new_position(seed):
    """Sequences built together (some share chunks inserted by an earlier
    sequence of the same call): rows start at each sequence's first newly
    stored token, so a shared chunk can be causal for one sequence and fully
    visible for another."""
    w = W.random_tree(seed, h=2, d=64, c=4, max_b=9, max_len=60, vocab=2)
    t = _tree(2, 64, 4)
    try:
        ids, slots = B.pkvt_tree_build(t, w.all_seq_tokens())
        q_from, pos = [], 0
        for u in range(w.b):
            L = w.seq_len(u)
            s = slots[pos:pos + L]
            new = np.nonzero(s >= 0)[0]
            q_from.append(int(new[0]) if new.size else L - 1)
            pos += L
        for ch in (0, 2):
            _check(t, ids, q_from, 4, 2, phase1_chunks=ch)
        # a subset, in another order, with rows from position 0
        order = [int(x) for x in np.random.default_rng(seed).permutation(ids)[: max(1, w.b // 2)]]
        _check(t, order, [0] * len(order), 4, 2)
    finally:
        B.pkvt_tree_destroy(t)


def test_chunked_prefill_plan():
    """A prompt fed in pieces: the first piece is stored, the second is
    appended; its rows see the first piece whole and themselves causally."""
    t = _tree(2, 64, 16)
    try:
        rng = np.random.default_rng(0)
        toks = rng.integers(0, 1000, size=150).astype(np.int32)
        ids, _ = B.pkvt_tree_build(t, [toks[:70]])
        B.pkvt_tree_append(t, [int(ids[0])] * 80, toks[70:])
        plan, info = _check(t, ids, [70], 16, 2)
        assert info["b"] == 80
    finally:
        B.pkvt_tree_destroy(t)


def test_prefill_plan_errors_and_staleness():
    t = _tree(2, 64, 16)
    try:
        ids, _ = B.pkvt_tree_build(t, [[1] * 40, [2] * 20])
        for args in [([int(ids[0])], [40]), ([int(ids[0])], [-1]), ([int(ids[0])] * 2, [0, 0])]:
            with pytest.raises(B.PkvtError) as e:
                B.pkvt_prefill_plan(t, *args)
            assert e.value.status == "INVALID_ARG"
        with pytest.raises(B.PkvtError) as e:
            B.pkvt_prefill_plan(t, [12345], [0])
        assert e.value.status == "UNKNOWN_SEQ"
        with pytest.raises(B.PkvtError) as e:
            B.pkvt_prefill_info_get(t)
        assert e.value.status == "STALE_PLAN"
        B.pkvt_prefill_plan(t, ids, [0, 0])
        B.pkvt_tree_append(t, [int(ids[0])], [3])
        with pytest.raises(B.PkvtError) as e:
            B.pkvt_prefill_upload(t, 0x1000, 1 << 20)
        assert e.value.status == "STALE_PLAN"
    finally:
        B.pkvt_tree_destroy(t)


def test_single_sequence_blocks_write_output_directly():
    """Sequences with many new rows: every block holds rows of one sequence
    and reads its whole visible path in one unit, so no row needs a merge."""
    pb = W.prefill_batch(5, 4, 96, 130, h=2, d=64, c=16, with_kv=False)
    t = _tree(2, 64, 16)
    try:
        B.pkvt_tree_build(t, [pb.w.segments[s].tokens for s in pb.residents])
        ids, _ = B.pkvt_tree_build(t, [pb.w.seq_tokens(u) for u in pb.seqs])
        plan, info = _check(t, ids, pb.q_from, 16, 2)
        assert info["slots"] == 0 and info["merge_rows"] == 0
        assert all(int(u[6]) == -1 for u in plan["units"])
    finally:
        B.pkvt_tree_destroy(t)


def test_heads_follow_dies():
    """With 8k heads, the units of head h run on workgroups g = h (mod 8)."""
    pb = W.prefill_batch(9, 6, 64, 40, h=16, d=64, c=16, with_kv=False)
    t = _tree(16, 64, 16)
    try:
        B.pkvt_tree_build(t, [pb.w.segments[s].tokens for s in pb.residents])
        ids, _ = B.pkvt_tree_build(t, [pb.w.seq_tokens(u) for u in pb.seqs])
        plan, _ = _check(t, ids, pb.q_from, 16, 16, workgroups=64)
        at = 0
        for g, (first, cnt) in enumerate(plan["wg_units"]):
            for k in range(first, first + cnt):
                assert int(plan["units"][k][3]) % 8 == g % 8
    finally:
        B.pkvt_tree_destroy(t)


def test_long_shared_prefix_takes_units_head_by_head():
    """When the chunks that many units re-read exceed a die's L2 for the die's
    heads (here a 4160-token prefix: 65 chunks x 64 KiB of K/V for its four
    heads, read by every unit), every workgroup of a die takes its units head
    by head: the older half of the die's workgroups in ascending head order
    (each with a share of every head of the die), the younger half (which
    start as the first finish) in descending order.  A short prefix keeps one
    head per workgroup here.  (Which rows and keys the units cover is checked
    by the other tests of this file and, on the GPU, by the prefill parity
    tests; this one looks at the order only.)"""
    for prefix, by_head in ((4160, True), (512, False)):
        pb = W.prefill_batch(11, 8, prefix, 256, h=32, d=64, c=64, with_kv=False)
        t = _tree(32, 64, 64)
        try:
            B.pkvt_tree_build(t, [pb.w.segments[s].tokens for s in pb.residents])
            ids, _ = B.pkvt_tree_build(t, [pb.w.seq_tokens(u) for u in pb.seqs])
            B.pkvt_prefill_plan(t, ids, pb.q_from, workgroups=64)
            plan = PV.parse(B.pkvt_prefill_blob(t))
            assert len(plan["units"]) == 8 * 32                # one unit per (sequence, head)
            per = 64 // 8
            for g, (first, cnt) in enumerate(plan["wg_units"]):
                heads = [int(plan["units"][k][3]) for k in range(first, first + cnt)]
                assert all(h % 8 == g % 8 for h in heads)
                if by_head:
                    older = g // 8 < per // 2
                    assert heads == (sorted(heads) if older else sorted(heads, reverse=True))
                    if older:
                        assert sorted(set(heads)) == [g % 8 + 8 * j for j in range(4)]
                else:
                    assert len(set(heads)) == 1
        finally:
            B.pkvt_tree_destroy(t)
