"""GPU parity of decode attention over token-granular trees
(PKVT_MATCH_TOKENS) against the fp64 oracle, and the K/V move kernel.

Under token matching a shared prefix that ends inside a chunk is stored once,
so paths hold partial chunks before their leaf (in shared and in private
parts), and prompts inserted by a later build call split nodes of an earlier
one, whose K/V then move (pkvt_kv_move) before the next attention call.
Workloads pass through workloads.unique_segment_starts so that equal token
prefixes always carry equal K/V.  Tolerance as for whole-chunk trees: max
|O_gpu - O_oracle| <= 2e-3.
"""
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
    out = ds.decode(layer)
    ds.torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _err(got, ref):
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.abs(got - ref).max())


def _partial_before_leaf(ds):
    from prefix_shared_kv_tree_amd import binding as B
    n = 0
    for i in ds.seq_ids:
        path = B.pkvt_tree_chunk_path(ds.tree, int(i))
        n += sum(B.pkvt_tree_chunk_fill(ds.tree, int(x)) < ds.w.c for x in path[:-1])
    return n


@pytest.mark.parametrize("seed", range(10))
def test_random_token_trees(seed):
    _torch()
    rng = np.random.default_rng(40 + seed)
    d = int(rng.choice([64, 128, 256]))
    c = int(rng.choice([16, 32, 64, 128]))
    h = int(rng.integers(1, 4))
    print(f"\n[case] token tree seed={seed} h={h} d={d} c={c}", flush=True)
    w = W.unique_segment_starts(W.random_tree(40 + seed, h=h, d=d, c=c, max_b=14, min_b=4,
                                              max_len=5 * c))
    ref = A.attention_batch(w)
    partial = 0
    for groups in (1, 3):
        for p1, p2, ms in [(0, 0, 0), (1, 1, 0), (0, 0, 1 << 20)]:
            ds = _setup(w, match="tokens", build_groups=groups, phase1_chunks=p1,
                        phase2_chunks=p2, min_share=ms)
            err = _err(_run(ds), ref)
            partial = max(partial, _partial_before_leaf(ds))
            print(f"[case]   groups={groups} p1={p1} p2={p2} min_share={ms} moves={ds.moves} "
                  f"partial_inside={_partial_before_leaf(ds)} err={err:.3e}", flush=True)
            assert err <= TOL
            ds.close()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_unaligned_shared_prompt(d):
    """40 sequences share a 1000-token prompt (chunk 64: 15 full chunks and a
    shared 40-token chunk, read by workgroup units whose keys end inside it),
    then private suffixes of 1..300 tokens; one prompt per build call, so the
    second call splits the first sequence's node at the end of the prompt
    and its tail K/V moves."""
    _torch()
    rng = np.random.default_rng(d)
    suffix = [int(x) for x in rng.integers(1, 301, size=40)]
    w = W.unique_segment_starts(W.one_prefix(600 + d, 40, 1000, suffix, h=2, d=d, c=64))
    ref = A.attention_batch(w)
    ds = _setup(w, match="tokens", build_groups=40)
    assert ds.moves == 64 - 1000 % 64
    err = _err(_run(ds), ref)
    print(f"\n[case] unaligned prompt d={d} moves={ds.moves} info={ds.info} err={err:.3e}", flush=True)
    assert err <= TOL
    assert ds.info["shared_chunks"] == 16 and ds.info["wg_units"] > 0
    assert ds.info["unique_tokens"] == 1000 + sum(suffix)
    ds.close()


def test_token_and_chunk_matching_agree():
    """The same workload under both matchings: the outputs agree within the
    tolerance, and token matching stores fewer tokens."""
    _torch()
    w = W.unique_segment_starts(W.layered_tree(77, 60, 3, h=2, d=128, c=32, max_chunks=4))
    ref = A.attention_batch(w)
    outs, uniq = {}, {}
    for match in ("chunks", "tokens"):
        ds = _setup(w, match=match, build_groups=2)
        outs[match] = _run(ds)
        uniq[match] = ds.info["unique_tokens"]
        print(f"\n[case] layered match={match} info={ds.info}", flush=True)
        assert _err(outs[match], ref) <= TOL
        ds.close()
    assert _err(outs["tokens"], outs["chunks"]) <= TOL
    assert uniq["tokens"] <= uniq["chunks"]


def _token_kv(torch, pool, slot, h, d, c, kind):
    """One token's [h, d] K or V read back through the documented pool
    layout: K slice [d/8][c][8]; V slice a run of blocks of F tokens (32, or
    16 when d is 256 or c is 16), each [d/16][F/8 groups][16][8]."""
    chunk, t = divmod(int(slot), c)
    base = chunk * h * c * d
    x = torch.arange(d, device=pool.device)
    paired = d <= 128 and c >= 32
    F = 32 if paired else 16
    w = t % F
    g = (w % 16) // 4 if paired else w // 8
    e = (w // 16) * 4 + w % 4 if paired else w % 8
    out = []
    for j in range(h):
        b = base + j * c * d
        if kind == "k":
            idx = b + ((x // 8) * c + t) * 8 + x % 8
        else:
            idx = b + (t - w) * d + (((x // 16) * (F // 8) + g) * 16 + x % 16) * 8 + e
        out.append(pool[idx])
    return torch.stack(out)


@pytest.mark.parametrize("d,c", [(64, 16), (128, 64), (256, 32)])
def test_kv_move_relocates_every_head(d, c):
    torch = _torch()
    from prefix_shared_kv_tree_amd import binding as B
    B.load()
    h, n_chunks = 3, 12
    t = B.pkvt_tree_create(h, d, c, n_chunks)
    try:
        elems = B.pkvt_pool_bytes(h, d, c, n_chunks) // 2
        g = torch.Generator(device="cuda")
        g.manual_seed(d + c)
        kp = torch.empty(elems, dtype=torch.float16, device="cuda").normal_(generator=g)
        vp = torch.empty(elems, dtype=torch.float16, device="cuda").normal_(generator=g)
        k0, v0 = kp.clone(), vp.clone()
        rng = np.random.default_rng(c)
        slots = rng.permutation(n_chunks * c)
        src, dst = slots[:40].astype(np.int64), slots[40:80].astype(np.int64)
        src[3] = -1                                      # skipped: out of range
        dst[5] = n_chunks * c                            # skipped: out of range
        sd = torch.from_numpy(src).cuda()
        dd = torch.from_numpy(dst).cuda()
        B.pkvt_kv_move(t, kp.data_ptr(), vp.data_ptr(), sd.data_ptr(), dd.data_ptr(), src.size,
                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for i, (s_, d_) in enumerate(zip(src, dst)):
            if i in (3, 5):
                continue
            for kind, new, old in (("k", kp, k0), ("v", vp, v0)):
                assert torch.equal(_token_kv(torch, new, d_, h, d, c, kind),
                                   _token_kv(torch, old, s_, h, d, c, kind))
        # every other slot is untouched
        moved = {int(x) for i, x in enumerate(dst) if i not in (3, 5)}
        for s_ in range(n_chunks * c):
            if s_ not in moved:
                for kind, new, old in (("k", kp, k0), ("v", vp, v0)):
                    assert torch.equal(_token_kv(torch, new, s_, h, d, c, kind),
                                       _token_kv(torch, old, s_, h, d, c, kind))
    finally:
        B.pkvt_tree_destroy(t)
