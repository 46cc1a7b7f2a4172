"""Decode-step query concat and cache insert on the GPU against the oracle:
bit-exact query rows and cache bytes (byte work, and for fp8 a code decided
in fp32 on both sides)."""
import numpy as np
import pytest
import torch

import oracle
from head_latent_attention_decode_amd import mla
from head_latent_attention_decode_amd import workloads as W

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _run(x, N):
    dev = torch.device("cuda:0")
    cache = x.cache.to(dev)
    kw = {}
    if x.cache_dtype == "fp8_e4m3fn":
        kw = dict(cache_scale_inv=torch.tensor([x.cache_scale_inv], dtype=torch.float32,
                                               device=dev),
                  cache_dtype="fp8_e4m3fn")
    q = mla.concat_q_insert_cache(x.ql_nope.to(dev), x.q_pe.to(dev), x.kv_c.to(dev),
                                  x.k_pe.to(dev), cache, x.slot_mapping.to(dev), **kw)
    torch.cuda.synchronize()
    return q.cpu(), cache.cpu()


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("T,N,nb,P,pad", [(1, 16, 3, 16, 0), (37, 128, 40, 64, 5),
                                          (256, 128, 300, 64, 0), (5, 0, 2, 16, 2)])
def test_insert_matches_oracle_bitwise(cache_dtype, T, N, nb, P, pad):
    x = W.make_insert_inputs(T, N, nb, P, seed=T * 7 + N, cache_dtype=cache_dtype, pad_every=pad)
    ref_cache = (_bits(x.cache) if cache_dtype == "bf16" else x.cache.numpy()).copy()
    ref_q = oracle.concat_insert(_bits(x.ql_nope), _bits(x.q_pe), _bits(x.kv_c),
                                 _bits(x.k_pe), x.slot_mapping.numpy(), ref_cache,
                                 x.cache_scale_inv)
    q, cache = _run(x, N)
    got_cache = _bits(cache) if cache_dtype == "bf16" else cache.numpy()
    assert (got_cache == ref_cache).all(), int((got_cache != ref_cache).sum())
    if N:
        assert (_bits(q) == ref_q).all()


def test_insert_fp8_covers_rounding_and_saturation():
    """Values at code midpoints, beyond 448 and tiny ones, through a scale of 1."""
    T, nb, P = 8, 2, 16
    x = W.make_insert_inputs(T, 1, nb, P, seed=99, cache_dtype="fp8_e4m3fn")
    codes = [c for c in range(0x7E)]
    vals = [oracle.e4m3fn_to_double(c) for c in codes]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    special = [500.0, 448.0, 1e4, 2.0 ** -12, 0.0, -0.0, -3.3, -600.0]
    pool = np.array(mids + [-m for m in mids] + special, dtype=np.float32)
    flat = torch.from_numpy(np.resize(pool, T * 576)).to(torch.bfloat16).view(T, 576)
    x.kv_c, x.k_pe = flat[:, :512].contiguous(), flat[:, 512:].contiguous()
    x.cache_scale_inv = 1.0
    ref_cache = x.cache.numpy().copy()
    oracle.concat_insert(_bits(x.ql_nope), _bits(x.q_pe), _bits(x.kv_c), _bits(x.k_pe),
                         x.slot_mapping.numpy(), ref_cache, 1.0)
    _, cache = _run(x, 1)
    assert (cache.numpy() == ref_cache).all(), int((cache.numpy() != ref_cache).sum())
