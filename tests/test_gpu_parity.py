"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerance: max |O_gpu - O_oracle| <= 2e-3 over every output element (fp16
Q/K/V, fp32 accumulation, fp16 output).  Special cases are exact where the
arithmetic makes them exact (a single key returns its V row bit for bit).
"""
import math
import os

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


def _setup(w, **kw):
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd.harness import DecodeSetup
    B.load()
    return DecodeSetup(w, **kw)


def _run(ds, layer=0):
    torch = ds.torch
    out = ds.decode(layer)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _err(got, ref):
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.abs(got - ref).max())


@pytest.mark.parametrize("name", ["tiny", "c2", "c3", "c4", "c5"])
@pytest.mark.parametrize("variant", ["tpp", "plain"])
def test_config_parity(name, variant):
    _torch()
    print(f"\n[case] config={name} variant={variant}", flush=True)
    w = W.make_config(name)
    ds = _setup(w, min_share=(1 << 20) if variant == "plain" else 0)
    got = _run(ds)
    ref = A.attention_batch(w)
    err = _err(got, ref)
    print(f"[case] config={name} variant={variant} max_abs_err={err:.3e} info={ds.info}", flush=True)
    assert err <= TOL
    if variant == "tpp" and name != "c5":
        assert ds.info["phase1_items"] > 0
    ds.close()


@pytest.mark.parametrize("seed", range(12))
def test_random_trees(seed):
    _torch()
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 256]))
    c = int(rng.choice([16, 32, 64, 128]))
    h = int(rng.integers(1, 4))
    print(f"\n[case] random tree seed={seed} h={h} d={d} c={c}", flush=True)
    w = W.random_tree(seed, h=h, d=d, c=c, max_b=12, max_len=5 * c)
    ref = A.attention_batch(w)
    for p1, p2, ms in [(0, 0, 0), (1, 1, 0), (3, 2, 3), (0, 0, 1 << 20)]:
        ds = _setup(w, phase1_chunks=p1, phase2_chunks=p2, min_share=ms)
        err = _err(_run(ds), ref)
        print(f"[case]   p1={p1} p2={p2} min_share={ms} err={err:.3e} info={ds.info}", flush=True)
        assert err <= TOL
        ds.close()


@pytest.mark.parametrize("seed", range(8))
def test_wide_trees(seed):
    """Many sequences per shared node, so phase-1 row blocks of 17..64 rows
    run as workgroup units (LDS-shared loads) and longer blocks are cut."""
    _torch()
    rng = np.random.default_rng(200 + seed)
    d = int(rng.choice([64, 128, 256]))
    c = int(rng.choice([16, 32, 64, 128]))
    h = int(rng.integers(1, 4))
    b = int(rng.integers(20, 141))
    n_roots = int(rng.integers(1, 4))
    print(f"\n[case] wide tree seed={seed} b={b} roots={n_roots} h={h} d={d} c={c}", flush=True)
    w = W.layered_tree(200 + seed, b, n_roots, h=h, d=d, c=c)
    ref = A.attention_batch(w)
    for p1, p2, ms in [(0, 0, 0), (1, 1, 0), (3, 2, 18)]:
        ds = _setup(w, phase1_chunks=p1, phase2_chunks=p2, min_share=ms)
        err = _err(_run(ds), ref)
        print(f"[case]   p1={p1} p2={p2} min_share={ms} err={err:.3e} info={ds.info}", flush=True)
        assert err <= TOL
        ds.close()


@pytest.mark.parametrize("rows", [17, 32, 33, 48, 64, 65, 81, 130])
@pytest.mark.parametrize("d,c,n_chunks", [(64, 16, 5), (128, 32, 3), (128, 64, 2), (256, 16, 3),
                                          (256, 128, 1)])
def test_unit_row_counts(rows, d, c, n_chunks):
    """One shared prefix read by `rows` sequences: unit row blocks of every
    size class, and prefixes whose length is not a multiple of 64 keys (the
    last step of a unit then has whole tiles past the end)."""
    _torch()
    print(f"\n[case] unit rows={rows} d={d} c={c} prefix_chunks={n_chunks}", flush=True)
    suffix = [(u * 7) % (2 * c) for u in range(rows)]
    w = W.one_prefix(300 + rows, rows, n_chunks * c, suffix, h=2, d=d, c=c)
    ref = A.attention_batch(w)
    ds = _setup(w, phase1_chunks=n_chunks)
    assert ds.info["wg_units"] > 0
    err = _err(_run(ds), ref)
    print(f"[case]   err={err:.3e} info={ds.info}", flush=True)
    assert err <= TOL
    ds.close()


def test_single_key_bit_exact():
    _torch()
    print("\n[case] single-key sequences", flush=True)
    w = W.random_tree(3, h=3, d=128, c=64, max_b=6, max_len=1)
    for p in w.seq_paths:
        assert sum(len(w.segments[s]) for s in p) == 1
    ds = _setup(w)
    got = ds.decode().cpu().numpy()
    for u in range(w.b):
        K, V = A.materialize(w, u)
        assert np.array_equal(got[u], V[0].astype(np.float16))
    ds.close()


def test_zero_query_gives_mean():
    _torch()
    w = W.make_config("c4")
    w.q[:] = 0
    ds = _setup(w)
    got = _run(ds)
    for u in [0, 17, 63]:
        _, V = A.materialize(w, u)
        assert np.abs(got[u] - V.mean(axis=0)).max() <= TOL
    ds.close()


def test_sharing_invariance():
    """Shared prefix vs the same K/V duplicated under distinct tokens."""
    _torch()
    w = W.make_config("c2")
    ref = A.attention_batch(w)
    ds1 = _setup(w)
    a = _run(ds1)
    assert ds1.info["phase1_items"] > 0
    ds1.close()
    wu = W.unshare(w)
    ds2 = _setup(wu)
    b = _run(ds2)
    assert ds2.info["phase1_items"] == 0 and ds2.info["shared_chunks"] == 0
    ds2.close()
    ea, eb = _err(a, ref), _err(b, ref)
    print(f"\n[case] sharing invariance shared={ea:.3e} duplicated={eb:.3e} "
          f"mutual={np.abs(a - b).max():.3e}", flush=True)
    assert ea <= TOL and eb <= TOL


def test_deterministic():
    _torch()
    w = W.make_config("c4")
    ds = _setup(w)
    a = ds.decode().clone()
    b = ds.decode().clone()
    ds.torch.cuda.synchronize()
    assert ds.torch.equal(a, b)
    ds.close()


def test_q_order_permutation():
    """Q/O rows follow q_order, whatever the depth-first order is."""
    torch = _torch()
    w = W.make_config("c4")
    ref = A.attention_batch(w)
    ds = _setup(w)
    perm = np.random.default_rng(0).permutation(w.b)
    order = ds.seq_ids[perm]
    ds.q = torch.from_numpy(np.ascontiguousarray(w.q[perm])).to("cuda")
    ds.replan(q_order=order)
    got = _run(ds)
    assert _err(got, ref[perm]) <= TOL
    # a subset of the live sequences
    sub = perm[:10]
    ds.q = torch.from_numpy(np.ascontiguousarray(w.q[sub])).to("cuda")
    ds.out = torch.empty_like(ds.q)
    ds.replan(q_order=ds.seq_ids[sub])
    got = _run(ds)
    assert _err(got, ref[sub]) <= TOL
    ds.close()


def test_layers_rotate():
    _torch()
    w = W.make_config("c2", layers=2)
    ds = _setup(w)
    for layer in range(2):
        assert _err(_run(ds, layer), A.attention_batch(w, layer=layer)) <= TOL
    ds.close()


def test_decode_append_and_lazy_upload():
    """Append tokens (K/V written by pkvt_kv_scatter), re-plan, upload only
    what changed, and match the oracle on the longer sequences."""
    torch = _torch()
    from prefix_shared_kv_tree_amd import binding as B
    w = W.make_config("tiny")
    ds = _setup(w, pool_slack=64)
    rng = np.random.default_rng(5)
    for step in range(40):
        toks = rng.integers(0, W.VOCAB, size=w.b).astype(np.int32)
        kn = rng.standard_normal((w.b, 1, w.h, w.d), dtype=np.float32).astype(np.float16)
        vn = rng.standard_normal((w.b, 1, w.h, w.d), dtype=np.float32).astype(np.float16)
        for u in range(w.b):
            w.segments.append(W.Segment(tokens=toks[u:u + 1], k=[kn[u]], v=[vn[u]]))
            w.seq_paths[u].append(len(w.segments) - 1)
        slots = B.pkvt_tree_append(ds.tree, ds.seq_ids, toks)
        sd = torch.from_numpy(slots).to("cuda")
        kd = torch.from_numpy(np.ascontiguousarray(kn[:, 0])).to("cuda")
        vd = torch.from_numpy(np.ascontiguousarray(vn[:, 0])).to("cuda")
        stream = torch.cuda.current_stream().cuda_stream
        B.pkvt_kv_scatter(ds.tree, ds.k_pools[0].data_ptr(), ds.v_pools[0].data_ptr(),
                          sd.data_ptr(), kd.data_ptr(), vd.data_ptr(), w.b, stream)
        mb, wb = B.pkvt_plan(ds.tree, ds.seq_ids)
        if mb > ds.meta_bytes or wb > ds.ws_bytes:
            ds.replan()
        else:
            B.pkvt_plan_upload(ds.tree, ds.meta.data_ptr(), ds.meta_bytes, stream)
        got = _run(ds)
        err = _err(got, A.attention_batch(w))
        assert err <= TOL, (step, err)
    ds.close()


@pytest.mark.parametrize("b,n_s,private", [(96, 2048, 56), (16, 2048, 8), (32, 1024, 1),
                                           (32, 4096, 960), (80, 2048, 40)])
def test_sweep_shapes_all_rows(b, n_s, private):
    """Full-size points of the divergence and batch sweeps (h = 32, d = 128,
    c = 64; b sequences sharing n_s prompt tokens plus `private` tokens
    each), two-phase and plain: every output row against the oracle (b = 80
    and 96 cut the shared rows into several blocks)."""
    _torch()
    w = W.one_prefix(4000 + b + n_s + private, b, n_s, private, h=32, d=128, c=64)
    ref = A.attention_batch(w)
    for variant, ms in (("tpp", 0), ("plain", 1 << 20)):
        print(f"\n[case] sweep shape b={b} n_s={n_s} private={private} {variant}", flush=True)
        ds = _setup(w, min_share=ms)
        err = _err(_run(ds), ref)
        print(f"[case]   all {b} rows err={err:.3e} info={ds.info}", flush=True)
        assert err <= TOL
        if variant == "tpp":
            assert ds.info["phase1_items"] > 0
        ds.close()


@pytest.mark.parametrize("d,c", [(256, 64), (256, 16), (256, 128), (64, 64)])
def test_head_dim_variants_long_prefix(d, c):
    """The long-shared-prompt batch (64 sequences, 4096 shared tokens,
    ragged private suffixes) at other head dims, with h d = 4096: every row
    against the oracle, two-phase and plain."""
    _torch()
    h = 4096 // d
    rng = np.random.default_rng(d + c)
    suffix = [int(x) for x in rng.integers(256, 1025, size=64)]
    print(f"\n[case] head_dim variant d={d} c={c} h={h}", flush=True)
    w = W.one_prefix(5000 + d + c, 64, 4096, suffix, h=h, d=d, c=c)
    ref = A.attention_batch(w)
    for ms in (0, 1 << 20):
        ds = _setup(w, min_share=ms)
        got = _run(ds)
        err = _err(got, ref)
        print(f"[case]   min_share={ms} all 64 rows err={err:.3e} info={ds.info}", flush=True)
        assert err <= TOL
        ds.close()


# ChunkAttention page, Knowl 6: b = 32 sequences of n_p context tokens each, the
# first n_s shared by all of them (h = 32, d = 128, c = 64, fp16).
@pytest.mark.parametrize("n_p,n_s", [(4096, 4096), (2048, 2048), (1024, 1024), (4096, 3072),
                                     (2048, 1024), (1024, 0)])
def test_knowl6_cells_all_rows(n_p, n_s):
    """Cells of the pages' microkernel grid, among them every fully shared
    corner (n_s = n_p: each context is one shared prompt), two-phase and
    plain: every output row against the oracle."""
    _torch()
    w = W.one_prefix(6000 + n_p + n_s, 32, n_s, n_p - n_s, h=32, d=128, c=64)
    assert all(w.seq_len(u) == n_p for u in range(32))
    ref = A.attention_batch(w)
    for variant, ms in (("tpp", 0), ("plain", 1 << 20)):
        print(f"\n[case] knowl6 n_p={n_p} n_s={n_s} {variant}", flush=True)
        ds = _setup(w, min_share=ms)
        err = _err(_run(ds), ref)
        print(f"[case]   all 32 rows err={err:.3e} info={ds.info}", flush=True)
        assert err <= TOL
        if variant == "tpp" and n_s > 0:
            assert ds.info["phase1_items"] > 0
        ds.close()


def test_single_key_bit_exact_head_dim_256():
    _torch()
    w = W.random_tree(3, h=2, d=256, c=16, max_b=6, max_len=1)
    for p in w.seq_paths:
        assert sum(len(w.segments[s]) for s in p) == 1
    ds = _setup(w)
    got = ds.decode().cpu().numpy()
    for u in range(w.b):
        K, V = A.materialize(w, u)
        assert np.array_equal(got[u], V[0].astype(np.float16))
    ds.close()


def test_items_of_64_chunks_and_long_private_contexts():
    """Items at the 64-chunk limit (one chunk id per lane, lane 63 used) and
    two sequences with ~20K private tokens each over a shared 4096-token
    prefix: many phase-2 pieces merged per row."""
    _torch()
    w = W.one_prefix(777, 3, 4096, [20000, 17, 12345], h=4, d=128, c=64)
    rows = [0, 1, 2]
    ref = A.attention_batch(w, seqs=rows)
    for p1, p2 in [(64, 64), (0, 0), (7, 3)]:
        ds = _setup(w, phase1_chunks=p1, phase2_chunks=p2)
        err = _err(_run(ds), ref)
        print(f"\n[case] long contexts p1={p1} p2={p2} err={err:.3e} info={ds.info}", flush=True)
        assert err <= TOL
        ds.close()


def test_many_sequences():
    """600 sequences in a three-level forest (many units, thousands of
    single-wave tasks and merges): every output row."""
    _torch()
    w = W.layered_tree(901, 600, 5, h=2, d=64, c=16, max_chunks=4)
    ref = A.attention_batch(w)
    ds = _setup(w)
    err = _err(_run(ds), ref)
    print(f"\n[case] 600 sequences err={err:.3e} info={ds.info}", flush=True)
    assert err <= TOL
    ds.close()
