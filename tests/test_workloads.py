"""The seeded input generators (CPU only): determinism and layout invariants."""
import numpy as np
import torch

from head_latent_attention_decode_amd import workloads as W


def test_deterministic():
    a = W.config_workload("tiny")
    b = W.config_workload("tiny")
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))
    assert torch.equal(a.cache.view(torch.int16), b.cache.view(torch.int16))
    assert torch.equal(a.block_table, b.block_table)


def test_layout_and_poison():
    wl = W.make_workload(4, 16, 16, [0, 1, 37, 100], seed=3, max_len=128)
    P = wl.page_size
    table = wl.block_table.numpy()
    lens = wl.seq_lens.numpy()
    poison = wl.meta["poison_block"]
    assert table.shape == (4, 8)
    used = []
    for b in range(4):
        pages = -(-int(lens[b]) // P)
        used.extend(table[b, :pages].tolist())
        assert (table[b, pages:] == poison).all()
    # physical pages: a permutation of 0..total-1, the poison page last
    assert sorted(used) == list(range(len(used)))
    assert poison == wl.cache.shape[0] - 1
    bits = wl.cache_bits()
    assert (bits[poison] == W.BF16_NAN_BITS).all()
    for b in range(4):
        L = int(lens[b])
        if L % P:
            last = table[b, (L - 1) // P]
            assert (bits[last, L % P:] == W.BF16_NAN_BITS).all()
            assert not (bits[last, : L % P] == W.BF16_NAN_BITS).all(axis=-1).any()


def test_ragged_lengths_in_range():
    lens = W.draw_seq_lens("uniform:1:32768", 128, 3)
    assert lens.min() >= 1 and lens.max() <= 32768 and lens.shape == (128,)


def test_fp8_cache_codes():
    wl = W.make_workload(2, 16, 16, [30, 45], seed=5, cache_dtype="fp8_e4m3fn")
    codes = wl.cache_bits()
    assert codes.dtype == np.uint8
    table = wl.block_table.numpy()
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    live = np.concatenate([vals[table[0, 0]], vals[table[0, 1], :14]])
    assert np.isfinite(live).all()
    # the largest magnitude maps to the top code (amax / scale = 448)
    allv = np.concatenate([vals[table[b, i]].ravel() for b in range(2) for i in range(3)
                           if table[b, i] != wl.meta["poison_block"]])
    assert np.nanmax(np.abs(allv)) == 448.0
    assert (codes[wl.meta["poison_block"]] == W.FP8_NAN_BITS).all()


def test_chunked_generation_matches_single_thread():
    a = W.make_workload(2, 16, 64, [40000, 3], seed=11, threads=1)
    b = W.make_workload(2, 16, 64, [40000, 3], seed=11, threads=4)
    assert torch.equal(a.cache.view(torch.int16), b.cache.view(torch.int16))
