"""Test helper: decode a plan blob (pkvt_plan_blob) and check it against the
tree's own paths.  Knows the blob layout documented in csrc/plan.h."""
from __future__ import annotations

from collections import defaultdict

import numpy as np

(H_MAGIC, H_SERIAL, H_B, H_NWAVES, H_NWG, H_NTASKS, H_NSLOTS, H_NMERGE, H_OFF_LISTS,
 H_OFF_TASKS, H_OFF_WAVES, H_OFF_CHUNKS, H_OFF_ROWS, H_OFF_MERGE, H_OFF_MPTR, H_OFF_MSLOTS,
 H_OFF_SEQLEN, H_TOTAL, H_NUNITS, H_OFF_WGUNITS, H_OFF_UNITS, H_OFF_QPOS) = range(22)
MAGIC = 0x504B5657
ROWS_PER_UNIT = 64
# rows of a prefill unit: 8 waves x 2 row tiles of 16 up to head_dim 128, 1 tile at 256
PREFILL_UNIT_ROWS = {64: 256, 128: 256, 256: 128}


def parse(blob: np.ndarray) -> dict:
    b = int(blob[H_B])
    nw, ng, nt = int(blob[H_NWAVES]), int(blob[H_NWG]), int(blob[H_NTASKS])
    waves = blob[blob[H_OFF_WAVES]:blob[H_OFF_WAVES] + nw * 8].reshape(nw, 8)
    chunks_base = int(blob[H_OFF_CHUNKS])
    mptr = blob[blob[H_OFF_MPTR]:blob[H_OFF_MPTR] + b + 1]
    nu = int(blob[H_NUNITS])
    units = blob[blob[H_OFF_UNITS]:blob[H_OFF_UNITS] + nu * 8].reshape(nu, 8)
    return dict(
        magic=int(blob[H_MAGIC]), b=b, n_slots=int(blob[H_NSLOTS]), n_wg=ng,
        wg_units=blob[blob[H_OFF_WGUNITS]:blob[H_OFF_WGUNITS] + ng * 2].reshape(ng, 2),
        units=units,
        unit_chunks=[blob[chunks_base + u[1]:chunks_base + u[1] + u[2]] for u in units],
        lists=blob[blob[H_OFF_LISTS]:blob[H_OFF_LISTS] + ng * 4 * 2].reshape(ng * 4, 2),
        tasks=blob[blob[H_OFF_TASKS]:blob[H_OFF_TASKS] + nt * 2].reshape(nt, 2),
        waves=waves,
        wave_chunks=[blob[chunks_base + w[0]:chunks_base + w[0] + w[1]] for w in waves],
        rows=blob[blob[H_OFF_ROWS]:blob[H_OFF_ROWS] + b],
        merge=blob[blob[H_OFF_MERGE]:blob[H_OFF_MERGE] + int(blob[H_NMERGE])],
        mptr=mptr,
        mslots=blob[blob[H_OFF_MSLOTS]:blob[H_OFF_MSLOTS] + int(mptr[-1])],
        seqlen=blob[blob[H_OFF_SEQLEN]:blob[H_OFF_SEQLEN] + b],
        qpos=blob[blob[H_OFF_QPOS]:blob[H_OFF_QPOS] + b] if blob[H_OFF_QPOS] else None,
        total=int(blob[H_TOTAL]),
    )


def check_plan(plan: dict, q_order, paths: dict, lens: dict, c: int, min_share: int = 2,
               max_rows: int = 16, heads: int = 1, unit_rows: int = 17, fills: dict = None):
    """paths / lens: seq id -> chunk path / token count (from the tree);
    fills: chunk id -> tokens stored (default: whole-chunk matching, every
    chunk before a leaf full).  Raises AssertionError on any violation."""
    assert plan["magic"] == MAGIC
    if fills is None:
        fills = {}
        for sid, path in paths.items():
            for k, x in enumerate(path):
                fills[int(x)] = c if k + 1 < len(path) else lens[sid] - c * (len(path) - 1)

    def start_of(path, k):
        """Sequence position of the first token of path[k]."""
        return sum(fills[int(y)] for y in path[:k])
    b = plan["b"]
    q_order = [int(x) for x in q_order]
    rows = [int(r) for r in plan["rows"]]
    assert sorted(rows) == list(range(b)), "rows is not a permutation"
    seq_at = [q_order[r] for r in rows]                  # depth-first position -> seq id
    for p in range(b):
        assert plan["seqlen"][p] == lens[seq_at[p]]
    # batch coverage of every chunk
    cover = defaultdict(set)
    for p in range(b):
        for x in paths[seq_at[p]]:
            cover[int(x)].add(p)
    # contiguity: the positions covering any chunk form one range
    for x, ps in cover.items():
        assert max(ps) - min(ps) + 1 == len(ps), f"chunk {x} covers a non-contiguous range"
    # every (position, path chunk) is visited exactly once
    seen = defaultdict(int)
    chunk_rows = defaultdict(set)
    slot_rows = {}
    direct = set()
    phase1 = []
    for wi, (w, ch) in enumerate(zip(plan["waves"], plan["wave_chunks"])):
        chunk_off, n_chunks, key_base, len_row, row_lo, n_rows, out, tail = [int(v) for v in w]
        assert n_chunks == len(ch) >= 1 and 1 <= n_rows <= max_rows
        multi = None
        for x in ch:
            x = int(x)
            for p in range(row_lo, row_lo + n_rows):
                assert x in [int(y) for y in paths[seq_at[p]]], "wave reads a chunk not on the row's path"
                seen[(p, x)] += 1
                chunk_rows[x].add(p)
            shared = len(cover[x]) >= min_share
            assert multi in (None, shared)
            multi = shared
        if not multi:
            assert n_rows == 1
        phase1.append(bool(multi))
        # key bound: only the wave that ends at the leaf uses the length
        p0 = row_lo
        path = [int(y) for y in paths[seq_at[p0]]]
        last = path.index(int(ch[-1]))
        # every chunk but the last is full (keys map to chunk k / c)
        for x in ch[:-1]:
            assert fills[int(x)] == c
        if last == len(path) - 1 and not multi:
            assert len_row == p0 and key_base == start_of(path, path.index(int(ch[0]))) and tail == 0
        else:
            assert len_row == -1
            assert n_chunks * c - tail == sum(fills[int(x)] for x in ch)
        if out < 0:
            assert n_rows == 1
            direct.add(row_lo)
        else:
            for r in range(n_rows):
                assert out + r not in slot_rows, "slot written twice"
                slot_rows[out + r] = row_lo + r
    # workgroup units: (row block, chunks) x every head exactly once; the row
    # blocks are the 64-row cuts of a phase-1 item with more than 16 rows
    unit_heads = defaultdict(list)
    wgu = plan["wg_units"]
    at = 0
    for g, (first, cnt) in enumerate(wgu):
        assert first == at and cnt >= 0
        at += cnt
    assert at == len(plan["units"])
    for u, ch in zip(plan["units"], plan["unit_chunks"]):
        n_keys, chunk_off, n_chunks, head, row_lo, n_rows, out, _ = [int(v) for v in u]
        assert n_chunks == len(ch) >= 1 and n_keys == sum(fills[int(x)] for x in ch)
        assert all(fills[int(x)] == c for x in ch[:-1])
        assert max(max_rows + 1, unit_rows) <= n_rows <= ROWS_PER_UNIT
        assert 0 <= head < heads and out >= 0
        unit_heads[(row_lo, n_rows, out, tuple(int(x) for x in ch))].append(head)
    for (row_lo, n_rows, out, ch), hs in unit_heads.items():
        assert sorted(hs) == list(range(heads)), "unit heads missing or repeated"
        for x in ch:
            assert len(cover[x]) >= min_share, "a unit reads an unshared chunk"
            for p in range(row_lo, row_lo + n_rows):
                assert x in [int(y) for y in paths[seq_at[p]]], "unit reads a chunk not on the row's path"
                seen[(p, x)] += 1
                chunk_rows[x].add(p)
        for r in range(n_rows):
            assert out + r not in slot_rows, "slot written twice"
            slot_rows[out + r] = row_lo + r
    for p in range(b):
        for x in paths[seq_at[p]]:
            assert seen.pop((p, int(x)), 0) == 1, f"chunk {x} of position {p} not visited once"
    assert not seen
    for x, ps in chunk_rows.items():
        assert ps == cover[x]
    # merge lists
    assert set(slot_rows) == set(range(plan["n_slots"]))
    merge = set(int(m) for m in plan["merge"])
    for p in range(b):
        sl = [int(s) for s in plan["mslots"][plan["mptr"][p]:plan["mptr"][p + 1]]]
        assert sorted(sl) == sorted(s for s, q in slot_rows.items() if q == p)
        if p in direct:
            assert not sl and p not in merge
        else:
            assert sl and p in merge
    # task lists: every (wave, head) exactly once; lists tile the task array
    lists = plan["lists"]
    assert lists.shape[0] == 4 * plan["n_wg"]
    at = 0
    lane_of = {}
    for lane, (first, cnt) in enumerate(lists):
        assert first == at and cnt >= 0
        for k in range(first, first + cnt):
            w, h = (int(x) for x in plan["tasks"][k])
            assert 0 <= h < heads
            assert (w, h) not in lane_of, "task listed twice"
            lane_of[(w, h)] = lane
        at += cnt
    assert at == len(plan["tasks"])
    assert set(lane_of) == {(w, h) for w in range(len(plan["waves"])) for h in range(heads)}
    # single-wave phase-1 tasks are the <= 16-row remainders of 64-row cuts
    for wi, w in enumerate(plan["waves"]):
        if phase1[wi]:
            assert int(w[5]) <= max_rows


def check_prefill_plan(plan: dict, seq_ids, q_from, paths: dict, lens: dict, c: int, heads: int,
                       d: int = 64, fills: dict = None):
    """Every prefill row (sequence s, position p) reads exactly the keys
    0 .. p of s, each once, from the chunks on s's path, in units of at most
    64 rows whose first key it can see; its partial slots are its merge list.
    fills: chunk id -> tokens stored (default: every chunk before a leaf
    full); a unit holds full chunks but its last."""
    if fills is None:
        fills = {}
        for sid, path in paths.items():
            for k, x in enumerate(path):
                fills[int(x)] = c if k + 1 < len(path) else lens[sid] - c * (len(path) - 1)
    R = plan["b"]
    rows_meta = []
    for s, a in zip(seq_ids, q_from):
        rows_meta += [(int(s), p) for p in range(int(a), lens[int(s)])]
    assert len(rows_meta) == R
    caller = [int(x) for x in plan["rows"]]
    assert sorted(caller) == list(range(R)), "rows is not a permutation"
    qpos = [int(x) for x in plan["qpos"]]
    for r in range(R):
        assert qpos[r] == rows_meta[caller[r]][1]
    assert len(plan["waves"]) == 0 and len(plan["tasks"]) == 0
    seen = defaultdict(lambda: defaultdict(int))        # (row, head) -> position -> count
    slot_rows = {}
    direct = defaultdict(int)                           # row -> units writing O directly (head 0)
    units_of = defaultdict(int)                         # row -> units reading it (head 0)
    for u, ch in zip(plan["units"], plan["unit_chunks"]):
        n_keys, chunk_off, n_chunks, head, row_lo, n_rows, out, key_base = [int(v) for v in u]
        assert 1 <= n_rows <= PREFILL_UNIT_ROWS[d] and 1 <= n_chunks <= 128 and 0 <= head < heads
        assert (n_keys + c - 1) // c == n_chunks
        assert all(fills[int(x)] == c for x in ch[:-1]) and n_keys <= sum(fills[int(x)] for x in ch)
        for i in range(n_rows):
            r = row_lo + i
            s, p = rows_meta[caller[r]]
            assert p >= key_base, "a row that sees none of the unit's keys"
            path = [int(x) for x in paths[s]]
            starts = [0]
            for x in path:
                starts.append(starts[-1] + fills[x])
            assert key_base in starts[:-1], "a unit that starts inside a chunk"
            k0 = starts.index(key_base)
            assert [int(x) for x in ch] == path[k0:k0 + n_chunks], "unit chunks are not on the row's path"
            for pos in range(key_base, min(key_base + n_keys, p + 1)):
                seen[(r, head)][pos] += 1
            if head == 0:
                units_of[r] += 1
                if out < 0:
                    direct[r] += 1
                else:
                    assert out + i not in slot_rows, "slot written twice"
                    slot_rows[out + i] = r
    for r in range(R):
        s, p = rows_meta[caller[r]]
        for h in range(heads):
            got = seen[(r, h)]
            assert sorted(got) == list(range(p + 1)), f"row {r} head {h} keys"
            assert all(v == 1 for v in got.values()), f"row {r} head {h} reads a key twice"
    assert set(slot_rows) == set(range(plan["n_slots"]))
    merge = [int(m) for m in plan["merge"]]
    assert merge == sorted(set(slot_rows.values())), "merge rows are the rows with partials"
    for r in range(R):
        sl = sorted(int(x) for x in plan["mslots"][plan["mptr"][r]:plan["mptr"][r + 1]])
        assert sl == sorted(k for k, v in slot_rows.items() if v == r)
        if direct[r]:
            assert direct[r] == 1 and units_of[r] == 1 and not sl, "a direct row reads one unit only"
        else:
            assert sl
