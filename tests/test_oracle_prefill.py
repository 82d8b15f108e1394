"""Pins for the prefill oracle (CPU only): a scalar brute force that walks
the segment list, a library implementation of masked attention (torch's
scaled_dot_product_attention in float64 with a causal or rectangular mask),
the position-0 special case, reduction of a sequence's last row to the
decode oracle, and causality (future keys cannot change a row)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from prefix_shared_kv_tree_amd import workloads as W


def _token_kv(w, u, t, hh):
    """K, V of token t of sequence u, head hh, found by walking u's segments."""
    for s in w.seq_paths[u]:
        seg = w.segments[s]
        if t < len(seg):
            return ([float(x) for x in seg.k[0][t, hh]], [float(x) for x in seg.v[0][t, hh]])
        t -= len(seg)
    raise IndexError


def _brute(w, u, p, qrow, hh, scale):
    qv = [float(x) for x in qrow[hh]]
    scores, vals = [], []
    for t in range(p + 1):
        k, v = _token_kv(w, u, t, hh)
        scores.append(math.fsum(a * b for a, b in zip(qv, k)) * scale)
        vals.append(v)
    m = max(scores)
    wts = [math.exp(s - m) for s in scores]
    tot = math.fsum(wts)
    return [math.fsum(wts[t] * vals[t][i] for t in range(p + 1)) / tot for i in range(len(qv))]


@pytest.mark.parametrize("seed", range(4))
def test_brute_force(seed):
    rng = np.random.default_rng(seed)
    pb = W.prefill_batch(seed, 3, int(rng.integers(0, 20)), [int(x) for x in rng.integers(1, 12, 3)],
                         h=2, d=4, c=4)
    O = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    scale = 1.0 / math.sqrt(pb.w.d)
    for r, (u, p) in enumerate(A.prefill_rows(pb.w, pb.seqs, pb.q_from)):
        for hh in range(pb.w.h):
            np.testing.assert_allclose(O[r, hh], _brute(pb.w, u, p, pb.q[r], hh, scale),
                                       rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("prefix,new", [(0, 37), (64, 30), (50, 9)])
def test_against_torch_masked_sdpa(prefix, new):
    """Rows q_from..L-1 of a sequence against keys 0..L-1 with key t visible
    to the row at position p iff t <= p (the causal mask when q_from = 0)."""
    pb = W.prefill_batch(11, 2, prefix, new, h=3, d=16, c=16)
    O = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    r0 = 0
    for u, a in zip(pb.seqs, pb.q_from):
        K, V = A.materialize(pb.w, u)
        L = K.shape[0]
        n = L - a
        q = torch.from_numpy(pb.q[r0:r0 + n].astype(np.float64).transpose(1, 0, 2).copy())  # [h, n, d]
        k = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))
        v = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))
        pos = torch.arange(a, L)[:, None]
        mask = torch.arange(L)[None, :] <= pos                                  # [n, L]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
        if a == 0:
            ref2 = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
            np.testing.assert_allclose(ref.numpy(), ref2.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(O[r0:r0 + n], ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)
        r0 += n


def test_position_zero_is_first_value_row():
    pb = W.prefill_batch(5, 2, 0, 7, h=2, d=8, c=4)
    O = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    r0 = 0
    for u in pb.seqs:
        _, V = A.materialize(pb.w, u)
        np.testing.assert_array_equal(O[r0], V[0])
        r0 += pb.w.seq_len(u)


def test_last_row_is_decode_attention():
    """The row of a sequence's last position sees the whole sequence: it is
    the decode attention of that sequence with the same query."""
    pb = W.prefill_batch(6, 4, 33, [3, 1, 8, 20], h=2, d=16, c=8)
    O = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    rows = A.prefill_rows(pb.w, pb.seqs, pb.q_from)
    for r, (u, p) in enumerate(rows):
        if p == pb.w.seq_len(u) - 1:
            K, V = A.materialize(pb.w, u)
            np.testing.assert_allclose(O[r], A.attention_one(pb.q[r], K, V, 0.25), rtol=1e-12, atol=1e-12)


def test_future_keys_do_not_matter():
    """Overwrite every key/value after a row's position with large values:
    that row's output must not move (a dropped causal mask would)."""
    pb = W.prefill_batch(8, 1, 20, 12, h=1, d=8, c=4)
    O = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    seg = pb.w.segments[pb.w.seq_paths[0][-1]]               # the new suffix
    seg.k[0][6:] = 30.0
    seg.v[0][6:] = -50.0
    O2 = A.prefill_attention(pb.w, pb.seqs, pb.q_from, pb.q)
    rows = A.prefill_rows(pb.w, pb.seqs, pb.q_from)
    for r, (_, p) in enumerate(rows):
        if p < 20 + 6:
            np.testing.assert_array_equal(O[r], O2[r])
        else:
            assert np.abs(O[r] - O2[r]).max() > 1e-4


def test_prefill_batch_rows():
    pb = W.prefill_batch(1, 3, 40, [5, 0, 20], h=2, d=16, c=16)
    assert pb.q_from == [32, 32, 32]
    assert pb.n_rows == (45 - 32) + (40 - 32) + (60 - 32)
    assert A.prefill_rows(pb.w, pb.seqs, pb.q_from)[:2] == [(0, 32), (0, 33)]
