"""Pins of the oracle's multi-token decode (uniform query length).

A brute-force softmax over the cache rows, written here directly in NumPy
from the page table, checks every query row on tiny contexts (causal and
not); q_len = 1 must be the single-token decode, and a non-causal row must
equal a single-token decode over the whole request.
"""
import numpy as np
import pytest
import torch

import oracle
from head_latent_attention_decode_amd import workloads as W


def _rows_of(wl, b):
    P = wl.page_size
    L = int(wl.seq_lens[b])
    bits = wl.cache.view(torch.int16).numpy().view(np.uint16)
    rows = []
    for t in range(L):
        blk = int(wl.block_table[b, t // P])
        rows.append([oracle.bf16_to_double(int(x)) for x in bits[blk, t % P]])
    return np.array(rows)


@pytest.mark.parametrize("causal", [True, False])
def test_multi_rows_brute_force(causal):
    QL, N = 3, 2
    wl = W.make_workload(3, N, 2, [3, 2, 5], seed=12)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(3, QL, N, 576, generator=g).to(torch.bfloat16).double().numpy()
    out, lse = oracle.mla_decode_multi(q, wl.cache.view(torch.int16).numpy().view(np.uint16),
                                       wl.block_table.numpy(), wl.seq_lens.numpy(),
                                       wl.softmax_scale, QL, causal=causal)
    for b in range(3):
        K = _rows_of(wl, b)
        L = K.shape[0]
        for j in range(QL):
            n_vis = L - (QL - 1 - j) if causal else L
            for n in range(N):
                if n_vis <= 0:
                    assert (out[b, j, n] == 0).all() and np.isneginf(lse[b, j, n])
                    continue
                s = wl.softmax_scale * (K[:n_vis] @ q[b, j, n])
                m = s.max()
                w = np.exp(s - m)
                ref_l = m + np.log(w.sum())
                ref_o = (w[:, None] * K[:n_vis, :512]).sum(0) / w.sum()
                assert abs(lse[b, j, n] - ref_l) <= 1e-12 * max(1.0, abs(ref_l))
                assert np.allclose(out[b, j, n], ref_o, rtol=1e-12, atol=1e-12)


def test_multi_q_len_one_and_noncausal_rows():
    wl = W.make_workload(2, 16, 16, [40, 9], seed=4)
    cache = wl.cache.view(torch.int16).numpy().view(np.uint16)
    q1 = wl.q.double().numpy()
    o1, l1 = oracle.mla_decode_multi(q1[:, None], cache, wl.block_table.numpy(),
                                     wl.seq_lens.numpy(), wl.softmax_scale, 1)
    ref_o, ref_l = oracle.mla_decode(oracle.Problem(q1, cache, wl.block_table.numpy(),
                                                    wl.seq_lens.numpy(), wl.softmax_scale))
    assert (o1[:, 0] == ref_o).all() and (l1[:, 0] == ref_l).all()
    q4 = np.repeat(q1[:, None], 4, axis=1)
    o4, l4 = oracle.mla_decode_multi(q4, cache, wl.block_table.numpy(), wl.seq_lens.numpy(),
                                     wl.softmax_scale, 4, causal=False)
    for j in range(4):
        assert (o4[:, j] == ref_o).all() and (l4[:, j] == ref_l).all()
