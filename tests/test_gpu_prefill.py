"""GPU parity of prefix-aware prefill (through the C ABI) against the fp64
prefill oracle: new query rows attend causally to the stored prefix and to
the new tokens up to themselves.  Tolerance as everywhere: max |O_gpu -
O_oracle| <= 2e-3."""
import math

import numpy as np
import pytest

from oracle import attention as A
from prefix_shared_kv_tree_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _setup(pb, **kw):
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd.harness import PrefillSetup
    B.load()
    return PrefillSetup(pb, **kw)


def _run(ps, layer=0):
    out = ps.run(layer)
    ps.torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all(), "non-finite output"
    return got


@pytest.mark.parametrize("b,prefix,new,d,c", [
    (1, 0, 40, 64, 16), (3, 40, [5, 1, 20], 64, 16), (20, 64, 17, 128, 16), (9, 100, 33, 128, 32),
    (70, 96, 3, 64, 32), (5, 200, [130, 1, 64, 65, 7], 128, 64), (4, 130, [70, 1, 129, 3], 256, 64),
    (6, 48, 40, 256, 16)])
def test_prefill_batch_all_rows(b, prefix, new, d, c):
    _torch()
    print(f"\n[case] prefill b={b} prefix={prefix} new={new} d={d} c={c}", flush=True)
    pb = W.prefill_batch(17 + b, b, prefix, new, h=2, d=d, c=c)
    ref = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    for ch in (0, 1):
        ps = _setup(pb, phase1_chunks=ch)
        err = float(np.abs(_run(ps) - ref).max())
        print(f"[case]   phase1_chunks={ch} err={err:.3e} info={ps.info}", flush=True)
        assert err <= TOL
        ps.close()


@pytest.mark.parametrize("prefix,new,c", [
    (0, 1, 64), (0, 64, 64), (64, 64, 64), (128, 64, 64), (192, 64, 64), (256, 64, 64),
    (300, 255, 64), (60, 200, 64), (0, 256, 64), (1, 511, 64), (100, 33, 32), (40, 129, 128),
    (17, 300, 16)])
def test_prefill_schedule_edges(prefix, new, c):
    """Head_dim 128 runs the ping-pong schedule: one sequence whose units have
    1 to 9 steps of 64 keys (the steps are unrolled by three and the last one
    is peeled) and 1 to 256 rows (waves without rows only load and wait),
    every row against the oracle."""
    _torch()
    print(f"\n[case] prefill schedule edges prefix={prefix} new={new} c={c}", flush=True)
    pb = W.prefill_batch(900 + prefix + new, 1, prefix, new, h=2, d=128, c=c)
    ref = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    ps = _setup(pb)
    err = float(np.abs(_run(ps) - ref).max())
    print(f"[case]   err={err:.3e} info={ps.info}", flush=True)
    assert err <= TOL
    ps.close()


@pytest.mark.parametrize("prefix,new,d,c", [
    (0, 1, 256, 64), (0, 16, 256, 64), (16, 16, 256, 64), (32, 16, 256, 64), (48, 16, 256, 64),
    (64, 16, 256, 64), (80, 16, 256, 64), (100, 28, 256, 32), (0, 128, 256, 16), (60, 77, 256, 128),
    (0, 1, 64, 64), (0, 64, 64, 64), (64, 64, 64, 64), (128, 64, 64, 64), (192, 64, 64, 64),
    (300, 255, 64, 64), (17, 200, 64, 16), (40, 129, 64, 128)])
def test_prefill_schedule_edges_other_head_dims(prefix, new, d, c):
    """Head_dim 256 takes four 16-key steps per barrier and head_dim 64 two
    64-key steps: one sequence whose units have 1 to 9 steps (every remainder
    of the groups of four and of two, and the alternation of the image
    pairs), every row against the oracle."""
    _torch()
    print(f"\n[case] prefill schedule edges prefix={prefix} new={new} d={d} c={c}", flush=True)
    pb = W.prefill_batch(950 + prefix + new + d, 1, prefix, new, h=2, d=d, c=c)
    ref = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    ps = _setup(pb)
    err = float(np.abs(_run(ps) - ref).max())
    print(f"[case]   err={err:.3e} info={ps.info}", flush=True)
    assert err <= TOL
    ps.close()


@pytest.mark.parametrize("b,prefix,new,d,c", [
    (12, 1000, [int(x) for x in np.random.default_rng(1).integers(1, 200, 12)], 128, 64),
    (7, 40, [3, 90, 17, 1, 64, 33, 5], 64, 16), (5, 130, [70, 1, 129, 3, 40], 256, 64)])
def test_prefill_token_matching(b, prefix, new, d, c):
    """Prefill over a token-granular tree: the stored prefix ends inside a
    chunk and is matched whole, so the new rows start at the prefix length,
    read the shared partial chunk through a unit that ends inside it, and
    their own chunks from a key base that is not a multiple of the chunk
    size."""
    _torch()
    print(f"\n[case] token prefill b={b} prefix={prefix} d={d} c={c}", flush=True)
    pb = W.prefill_batch(57 + b, b, prefix, new, h=2, d=d, c=c, match="tokens")
    assert pb.q_from == [prefix] * b
    ref = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    for ch in (0, 1):
        ps = _setup(pb, phase1_chunks=ch, match="tokens")
        err = float(np.abs(_run(ps) - ref).max())
        print(f"[case]   phase1_chunks={ch} err={err:.3e} info={ps.info}", flush=True)
        assert err <= TOL
        ps.close()


def test_prefill_first_row_is_value_row_bit_exact():
    """A sequence prefilled from position 0: its first row sees one key, so
    its output is that key's V row exactly."""
    _torch()
    pb = W.prefill_batch(3, 4, 0, [9, 1, 30, 17], h=3, d=128, c=16)
    ps = _setup(pb)
    got = ps.run().cpu().numpy()
    r = 0
    for u in pb.seqs:
        _, V = A.materialize(pb.w, u)
        assert np.array_equal(got[r], V[0].astype(np.float16))
        r += pb.w.seq_len(u)
    ps.close()


@pytest.mark.parametrize("layers", [2])
def test_prefill_full_size_sampled(layers):
    """32 sequences arriving over a stored 1024-token prefix with 512 new
    tokens each (h = 32, d = 128, c = 64): sampled rows of both layers."""
    _torch()
    pb = W.prefill_batch(1001, 32, 1024, 512, h=32, d=128, c=64, layers=layers)
    ps = _setup(pb)
    rows = [0, 1, 63, 64, 511, 512, 4095, 9000, pb.n_rows - 1]
    for l in range(layers):
        got = _run(ps, l)
        ref = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q, layer=l, rows=rows)
        err = float(np.abs(got[rows] - ref[rows]).max())
        print(f"\n[case] prefill full size layer {l} err={err:.3e} info={ps.info}", flush=True)
        assert err <= TOL
    ps.close()


@pytest.mark.parametrize("seed", range(6))
def test_prefill_random_trees_batch_internal_sharing(seed):
    """Sequences inserted in one call, later ones matching chunks an earlier
    one stores in the same call: every sequence's rows start at its first
    newly stored token."""
    torch = _torch()
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd.harness import gather_new_tokens
    B.load()
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 256]))
    c = int(rng.choice([16, 32, 64]))
    w = W.random_tree(600 + seed, h=2, d=d, c=c, max_b=10, max_len=4 * c, vocab=2)
    tree = B.pkvt_tree_create(w.h, w.d, w.c, sum(-(-w.seq_len(u) // c) for u in range(w.b)) + 4)
    try:
        ids, slots = B.pkvt_tree_build(tree, w.all_seq_tokens())
        q_from, pos = [], 0
        for u in range(w.b):
            L = w.seq_len(u)
            new = np.nonzero(slots[pos:pos + L] >= 0)[0]
            q_from.append(int(new[0]) if new.size else L - 1)
            pos += L
        elems = B.pkvt_pool_bytes(w.h, w.d, w.c, B.pkvt_tree_stats(tree)["capacity"]) // 2
        kp = torch.zeros(elems, dtype=torch.float16, device="cuda")
        vp = torch.zeros(elems, dtype=torch.float16, device="cuda")
        k_new, v_new, s_new = gather_new_tokens(w, slots, 0)
        stream = torch.cuda.current_stream().cuda_stream
        kd, vd = torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda()
        sd = torch.from_numpy(s_new).cuda()
        B.pkvt_kv_scatter(tree, kp.data_ptr(), vp.data_ptr(), sd.data_ptr(), kd.data_ptr(),
                          vd.data_ptr(), s_new.size, stream)
        R = sum(w.seq_len(u) - a for u, a in enumerate(q_from))
        q = np.random.default_rng(seed + 50).standard_normal((R, w.h, w.d), dtype=np.float32).astype(np.float16)
        qd = torch.from_numpy(q).cuda()
        out = torch.empty_like(qd)
        mb, wb = B.pkvt_prefill_plan(tree, ids, q_from)
        meta = torch.empty(mb // 4, dtype=torch.int32, device="cuda")
        ws = torch.empty(wb // 4, dtype=torch.float32, device="cuda")
        B.pkvt_prefill_upload(tree, meta.data_ptr(), mb, stream)
        B.pkvt_prefill_attn(tree, meta.data_ptr(), qd.data_ptr(), kp.data_ptr(), vp.data_ptr(),
                            out.data_ptr(), ws.data_ptr(), wb, 1.0 / math.sqrt(w.d), stream)
        torch.cuda.synchronize()
        ref = A.prefill_attention(w, list(range(w.b)), q_from, q)
        err = float(np.abs(out.float().cpu().numpy() - ref).max())
        print(f"\n[case] prefill random tree seed={seed} d={d} c={c} rows={R} err={err:.3e}", flush=True)
        assert err <= TOL
    finally:
        B.pkvt_tree_destroy(tree)


def test_chunked_prefill_matches_whole_prefill():
    """A prompt fed in two pieces (the second appended after the first is
    stored) gives, for the second piece's rows, the result of feeding it
    whole -- the exactness of chunked prefill -- both within tolerance of
    the oracle."""
    torch = _torch()
    from prefix_shared_kv_tree_amd import binding as B
    B.load()
    h, d, c, L, a = 4, 128, 32, 300, 137
    pb = W.prefill_batch(77, 1, 0, L, h=h, d=d, c=c)
    w = pb.w
    K = w.segments[w.seq_paths[0][0]].k[0]
    V = w.segments[w.seq_paths[0][0]].v[0]
    toks = w.seq_tokens(0)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    ref = A.prefill_attention(w, [0], [0], pb.q)

    def prefill(tree, ids, kp, vp, q_from, q):
        qd = torch.from_numpy(np.ascontiguousarray(q)).cuda()
        out = torch.empty_like(qd)
        mb, wb = B.pkvt_prefill_plan(tree, ids, [q_from])
        meta = torch.empty(mb // 4, dtype=torch.int32, device="cuda")
        ws = torch.empty(wb // 4, dtype=torch.float32, device="cuda")
        B.pkvt_prefill_upload(tree, meta.data_ptr(), mb, stream)
        B.pkvt_prefill_attn(tree, meta.data_ptr(), qd.data_ptr(), kp.data_ptr(), vp.data_ptr(),
                            out.data_ptr(), ws.data_ptr(), wb, scale, stream)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)

    def write(tree, kp, vp, slots, k, v):
        sd = torch.from_numpy(np.ascontiguousarray(slots)).cuda()
        kd = torch.from_numpy(np.ascontiguousarray(k)).cuda()
        vd = torch.from_numpy(np.ascontiguousarray(v)).cuda()
        B.pkvt_kv_scatter(tree, kp.data_ptr(), vp.data_ptr(), sd.data_ptr(), kd.data_ptr(),
                          vd.data_ptr(), slots.size, stream)

    results = []
    for pieces in ([(0, L)], [(0, a), (a, L)]):
        tree = B.pkvt_tree_create(h, d, c, 64)
        try:
            elems = B.pkvt_pool_bytes(h, d, c, 64) // 2
            kp = torch.zeros(elems, dtype=torch.float16, device="cuda")
            vp = torch.zeros(elems, dtype=torch.float16, device="cuda")
            got = np.full((L, h, d), np.nan)
            ids = None
            for lo, hi in pieces:
                if ids is None:
                    ids, slots = B.pkvt_tree_build(tree, [toks[lo:hi]])
                else:
                    slots = B.pkvt_tree_append(tree, [int(ids[0])] * (hi - lo), toks[lo:hi])
                write(tree, kp, vp, slots, K[lo:hi], V[lo:hi])
                got[lo:hi] = prefill(tree, ids, kp, vp, lo, pb.q[lo:hi])
            assert float(np.abs(got - ref).max()) <= TOL
            results.append(got)
        finally:
            B.pkvt_tree_destroy(tree)
    print(f"\n[case] chunked vs whole prefill: max diff {np.abs(results[0] - results[1]).max():.3e}",
          flush=True)
    assert float(np.abs(results[0] - results[1]).max()) <= 2 * TOL


@pytest.mark.parametrize("d,c,prefix,new", [(128, 16, 90 * 16 + 5, [40, 300]), (64, 16, 1700, 70),
                                            (256, 16, 1500, [3, 64])])
def test_prefill_units_over_64_chunks(d, c, prefix, new):
    """Rows whose visible path is longer than 64 chunks: a unit reads up to
    128 chunks, its chunk ids held in two registers per lane."""
    _torch()
    b = 1 if np.isscalar(new) else len(new)
    pb = W.prefill_batch(31 + d, b, prefix, new, h=2, d=d, c=c)
    ps = _setup(pb)
    blob_units = ps.info["wg_units"]
    err = float(np.abs(_run(ps) - A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)).max())
    print(f"\n[case] prefill > 64 chunks d={d} c={c} prefix={prefix} new={new} err={err:.3e} "
          f"units={blob_units}", flush=True)
    assert err <= TOL
    ps.close()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_prefill_grid_size_does_not_change_results(d):
    """One prefill workgroup is resident per compute unit; a grid larger than
    that is dispatched as workgroups finish.  Every unit's arithmetic and the
    merge order are fixed by the plan, not by which workgroup runs a unit, so
    grids of 256, 512 and 1024 workgroups give bit-identical outputs (and
    match the oracle)."""
    _torch()
    print(f"\n[case] prefill grid sizes d={d}", flush=True)
    pb = W.prefill_batch(61 + d, 24, 300, [int(x) for x in np.random.default_rng(d).integers(1, 400, 24)],
                         h=3, d=d, c=32)
    ref = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    ps = _setup(pb)
    outs = []
    for g in (256, 512, 1024):
        ps.replan(workgroups=g)
        outs.append(_run(ps))
        print(f"[case]   workgroups={g} err={float(np.abs(outs[-1] - ref).max()):.3e} "
              f"units={ps.info['wg_units']} slots={ps.info['slots']}", flush=True)
    ps.close()
    assert float(np.abs(outs[0] - ref).max()) <= TOL
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
