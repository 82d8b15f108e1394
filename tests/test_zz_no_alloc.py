"""pkvt_attn_decode_noalloc: decode attention with the partials in the
library's fixed device scratch instead of a caller workspace (for callers
that cannot allocate).  Checked through the C ABI against pkvt_attn_decode
on the same plan, twice in a row (the second call on a smaller batch, so the
scratch holds the first call's partials), and against the fp64 oracle."""
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


def _both(ds):
    """O from pkvt_attn_decode (workspace) and from the no-allocation entry
    point, same tree, plan and inputs."""
    from prefix_shared_kv_tree_amd import binding as B
    torch = ds.torch
    stream = torch.cuda.current_stream().cuda_stream
    ws = ds.ws.data_ptr() if ds.ws_bytes else 0
    out_ws = torch.full_like(ds.q, float("nan"))
    out_na = torch.full_like(ds.q, float("nan"))
    B.pkvt_attn_decode(ds.tree, ds.meta.data_ptr(), ds.q.data_ptr(), ds.k_pools[0].data_ptr(),
                       ds.v_pools[0].data_ptr(), out_ws.data_ptr(), ws, ds.ws_bytes, ds.scale,
                       stream)
    B.pkvt_attn_decode_noalloc(ds.tree, ds.meta.data_ptr(), ds.q.data_ptr(),
                               ds.k_pools[0].data_ptr(), ds.v_pools[0].data_ptr(),
                               out_na.data_ptr(), ds.scale, stream)
    torch.cuda.synchronize()
    return out_ws.cpu().numpy(), out_na.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice():
    _torch()
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd.harness import DecodeSetup
    B.load()
    # first call: 32 sequences over a 1024-token shared prefix (partials for
    # every row); second: a smaller two-level batch
    cases = [W.one_prefix(71, 32, 1024, [int(x) for x in np.random.default_rng(1).integers(1, 300, 32)],
                          h=8, d=128, c=64),
             W.layered_tree(72, 12, 2, h=4, d=128, c=64, max_chunks=5)]
    for i, w in enumerate(cases):
        print(f"\n[case] noalloc call {i}: b={w.b} h={w.h}", flush=True)
        ds = DecodeSetup(w)
        assert ds.ws_bytes > 0 and ds.info["merge_rows"] > 0
        got_ws, got_na = _both(ds)
        ref = A.attention_batch(w)
        err = float(np.abs(got_na.astype(np.float64) - ref).max())
        print(f"[case]   workspace bytes {ds.ws_bytes}, max abs err {err:.3e}", flush=True)
        assert np.isfinite(got_na).all()
        assert np.array_equal(got_ws.view(np.uint16), got_na.view(np.uint16))
        assert err <= TOL
        ds.close()


def test_noalloc_rejects_plans_beyond_the_scratch():
    """A plan whose partials exceed the fixed scratch is refused before any
    launch (BUFFER_TOO_SMALL); the workspace entry point still serves it."""
    _torch()
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd.harness import DecodeSetup
    B.load()
    w = W.one_prefix(73, 64, 4096, 64, h=32, d=128, c=64)
    ds = DecodeSetup(w, phase1_chunks=1)          # 64 items x 64 rows of partials
    assert ds.ws_bytes > B.PKVT_NOALLOC_SCRATCH_BYTES
    with pytest.raises(B.PkvtError) as e:
        B.pkvt_attn_decode_noalloc(ds.tree, ds.meta.data_ptr(), ds.q.data_ptr(),
                                   ds.k_pools[0].data_ptr(), ds.v_pools[0].data_ptr(),
                                   ds.out.data_ptr(), ds.scale,
                                   ds.torch.cuda.current_stream().cuda_stream)
    assert e.value.status == "BUFFER_TOO_SMALL"
    got = ds.decode(0)
    ds.torch.cuda.synchronize()
    rows = [0, 31, 63]
    ref = A.attention_batch(w, seqs=rows)
    assert float(np.abs(got.float().cpu().numpy()[rows] - ref[rows]).max()) <= TOL
    ds.close()
