"""GPU parity of the decode loop: per step, joins (departure + arrival),
one appended token per row written by pkvt_kv_scatter, lazy plan refresh and
upload, attention for every layer -- against the fp64 oracle on the batch the
step sees (ChunkAttention page, Knowl 1 decoding iteration, arrival and
departure; Knowl 5 lazy context copy).  Same tolerance as every parity test:
max |O_gpu - O_oracle| <= 2e-3."""
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


def _loop(tr, layers):
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd.harness import DecodeLoop, DecodeSetup, loop_pool_chunks
    B.load()
    ds = DecodeSetup(tr.base, layers=layers, pool_chunks=loop_pool_chunks(tr))
    return ds, DecodeLoop(ds, tr)


def _check(loop, tr, t, layers, rows=None):
    torch = loop.torch
    torch.cuda.synchronize()
    got = loop.out.float().cpu().numpy().astype(np.float64)
    wt = tr.workload_at(t)
    worst = 0.0
    for l in range(layers):
        ref = A.attention_batch(wt, layer=l, seqs=rows)
        g = got[l]
        if rows is not None:
            g, ref = g[list(rows)], ref[list(rows)]
        assert np.isfinite(g).all()
        err = float(np.abs(g - ref).max())
        worst = max(worst, err)
        assert err <= TOL, (t, l, err)
    return worst


def test_decode_loop_every_step_small():
    """Four rows over a shared 64-token root, 2 layers, a join every 5 steps:
    every step's output of every layer."""
    _torch()
    print("\n[case] decode loop tiny: 60 steps, churn 5, 2 layers", flush=True)
    w = W.make_config("tiny", layers=2)
    tr = W.decode_trace(w, 60, seed=21, churn_every=5)
    ds, loop = _loop(tr, 2)
    worst = 0.0
    for t in range(tr.steps):
        loop.step(t)
        worst = max(worst, _check(loop, tr, t, 2))
    print(f"[case]   worst err {worst:.3e} host counts {loop.host.count}", flush=True)
    assert loop.host.count["plan_full"] >= tr.steps // w.c
    ds.close()


@pytest.mark.parametrize("seed,d,c", [(31, 128, 32), (32, 64, 16), (33, 128, 64), (34, 256, 32)])
def test_decode_loop_unaligned_prefix(seed, d, c):
    """A shared prefix that ends inside a chunk (its tail is private to each
    sequence, and a new arrival writes it again), ragged suffixes, joins every
    6 steps."""
    _torch()
    rng = np.random.default_rng(seed)
    b = 24
    prefix = 3 * c + int(rng.integers(1, c))
    suffix = [int(x) for x in rng.integers(0, 3 * c, size=b)]
    print(f"\n[case] decode loop unaligned seed={seed} d={d} c={c} prefix={prefix}", flush=True)
    w = W.one_prefix(seed, b, prefix, suffix, h=3, d=d, c=c)
    tr = W.decode_trace(w, 2 * c + 5, seed=seed, churn_every=6, suffix=(1, 2 * c))
    ds, loop = _loop(tr, 1)
    worst = 0.0
    for t in range(tr.steps):
        loop.step(t)
        if t % 4 == 0 or t == tr.steps - 1:
            worst = max(worst, _check(loop, tr, t, 1))
    print(f"[case]   worst err {worst:.3e} host counts {loop.host.count}", flush=True)
    ds.close()


@pytest.mark.parametrize("seed,d,c", [(41, 128, 32), (42, 64, 16), (43, 256, 64)])
def test_decode_loop_token_matching(seed, d, c):
    """The loop over a token-granular tree: a shared prompt that ends inside
    a chunk is stored once (the batch arrives one prompt per build call: the second
    calls split earlier nodes and their K/V move), decode appends fill the
    split leaves, joins every 5 steps; every step against the oracle."""
    _torch()
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd.harness import DecodeLoop, DecodeSetup, loop_pool_chunks
    B.load()
    rng = np.random.default_rng(seed)
    b = 12
    prefix = 2 * c + int(rng.integers(1, c))
    suffix = [int(x) for x in rng.integers(1, 2 * c, size=b)]
    print(f"\n[case] decode loop token matching seed={seed} d={d} c={c} prefix={prefix}", flush=True)
    w = W.unique_segment_starts(W.one_prefix(seed, b, prefix, suffix, h=2, d=d, c=c))
    tr = W.decode_trace(w, c + 9, seed=seed, churn_every=5, suffix=(1, 2 * c), unique_starts=True)
    ds = DecodeSetup(w, layers=1, pool_chunks=loop_pool_chunks(tr) + b, match="tokens",
                     build_groups=b)
    assert ds.moves > 0
    loop = DecodeLoop(ds, tr)
    worst = 0.0
    for t in range(tr.steps):
        loop.step(t)
        worst = max(worst, _check(loop, tr, t, 1))
    print(f"[case]   moves {ds.moves} worst err {worst:.3e} host counts {loop.host.count}", flush=True)
    ds.close()


def test_decode_loop_long_prefix_sampled():
    """The 4096-token shared prefix batch of 64 (head_dim 128, chunk 64,
    32 heads), 40 steps with a join every 8: sampled rows, including the
    rows that were replaced, at three steps."""
    _torch()
    print("\n[case] decode loop c3: 40 steps, churn 8", flush=True)
    w = W.make_config("c3")
    tr = W.decode_trace(w, 40, seed=1002, churn_every=8, suffix=(256, 1024))
    ds, loop = _loop(tr, 1)
    joined = sorted({j.row for j in tr.joins})
    rows = sorted(set([0, 31, 63] + joined))
    worst = 0.0
    for t in range(tr.steps):
        loop.step(t)
        if t in (0, 17, tr.steps - 1):
            worst = max(worst, _check(loop, tr, t, 1, rows=rows))
    print(f"[case]   rows {rows} worst err {worst:.3e} host counts {loop.host.count}", flush=True)
    ds.close()


@pytest.mark.parametrize("d,c,n", [(128, 64, 64), (64, 16, 256), (128, 32, 1), (256, 128, 100)])
def test_scatter_host_slots_matches_device_slots(d, c, n):
    """pkvt_kv_scatter_host_slots (slots in the launch arguments) writes the
    same pool bytes as pkvt_kv_scatter (slots in device memory), skipping
    -1 and out-of-pool entries alike."""
    torch = _torch()
    from prefix_shared_kv_tree_amd import binding as B
    B.load()
    h, pool = 3, 40
    tree = B.pkvt_tree_create(h, d, c, pool)
    try:
        rng = np.random.default_rng(n)
        slots = rng.choice(pool * c, size=n, replace=False).astype(np.int64)
        slots[1::7] = -1
        if n > 3:
            slots[3] = pool * c + 5                      # outside the pool: skipped
        kn = torch.from_numpy(rng.standard_normal((n, h, d), dtype=np.float32).astype(np.float16)).cuda()
        vn = torch.from_numpy(rng.standard_normal((n, h, d), dtype=np.float32).astype(np.float16)).cuda()
        elems = B.pkvt_pool_bytes(h, d, c, pool) // 2
        pools = [torch.zeros(elems, dtype=torch.float16, device="cuda") for _ in range(4)]
        stream = torch.cuda.current_stream().cuda_stream
        sd = torch.from_numpy(slots).cuda()
        B.pkvt_kv_scatter(tree, pools[0].data_ptr(), pools[1].data_ptr(), sd.data_ptr(),
                          kn.data_ptr(), vn.data_ptr(), n, stream)
        host = slots.copy()
        B.pkvt_kv_scatter_host_slots(tree, pools[2].data_ptr(), pools[3].data_ptr(), host,
                                     kn.data_ptr(), vn.data_ptr(), stream)
        host[:] = -1                                     # reusable as soon as the call returns
        torch.cuda.synchronize()
        assert torch.equal(pools[0], pools[2]) and torch.equal(pools[1], pools[3])
        assert int((pools[0] != 0).sum()) > 0
        with pytest.raises(B.PkvtError):
            B.pkvt_kv_scatter_host_slots(tree, pools[2].data_ptr(), pools[3].data_ptr(),
                                         np.zeros(B.PKVT_INLINE_SLOTS + 1, np.int64),
                                         kn.data_ptr(), vn.data_ptr(), stream)
    finally:
        B.pkvt_tree_destroy(tree)
