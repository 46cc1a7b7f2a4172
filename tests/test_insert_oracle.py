"""Pins of the oracle's E4M3FN encoder and of its decode-step insert + concat.

The encoder is checked against the code table (every finite code is its own
nearest value), against exact midpoints (ties go to the even code), against
saturation, and against a library routine (torch's float8_e4m3fn cast of
values already inside the finite range).  The insert is checked by
properties that hold whatever the arithmetic: the query rows are the two
inputs side by side, each row lands at its slot's page and row, padding
tokens and out-of-range slots write nothing, and an fp8 row decodes back to
within half a code step of the input.
"""
import numpy as np
import pytest
import torch

import oracle
from head_latent_attention_decode_amd import workloads as W



def _finite_codes():
    return [c for c in range(256) if np.isfinite(oracle.e4m3fn_to_double(c))]


def test_encoder_roundtrips_every_finite_code():
    for c in _finite_codes():
        v = oracle.e4m3fn_to_double(c)
        e = oracle.e4m3fn_from_float(v)
        if v == 0.0:
            assert e in (0x00, 0x80) and (e >> 7) == (1 if np.signbit(v) else 0)
        else:
            assert e == c, (c, v, e)


def test_encoder_ties_go_to_even_code():
    pos = [c for c in _finite_codes() if c < 0x7F]
    for lo, hi in zip(pos[:-1], pos[1:]):
        a, b = oracle.e4m3fn_to_double(lo), oracle.e4m3fn_to_double(hi)
        mid = np.float32((a + b) / 2)
        if float(mid) != (a + b) / 2:       # not representable in fp32: no exact tie
            continue
        want = lo if lo % 2 == 0 else hi
        assert oracle.e4m3fn_from_float(float(mid)) == want, (lo, hi)
        assert oracle.e4m3fn_from_float(-float(mid)) == want | 0x80


def test_encoder_saturates_and_keeps_nan():
    for v in (448.0, 449.0, 464.0, 1e6, 3.0e38):
        assert oracle.e4m3fn_from_float(v) == 0x7E
        assert oracle.e4m3fn_from_float(-v) == 0xFE
    assert oracle.e4m3fn_from_float(float("nan")) == 0x7F


def test_encoder_matches_torch_cast_inside_range():
    g = torch.Generator().manual_seed(5)
    x = torch.cat([torch.randn(4000, generator=g) * s for s in (0.01, 1.0, 30.0, 200.0)])
    x = x.clamp(-448, 448)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3fn_from_float(float(v)) for v in x.numpy()], dtype=np.uint8)
    assert (ref == mine).all()


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8_e4m3fn"])
def test_insert_oracle_properties(cache_dtype):
    T, N, nb, P = 9, 3, 5, 4
    x = W.make_insert_inputs(T, N, nb, P, seed=3, cache_dtype=cache_dtype, pad_every=4)
    slots = x.slot_mapping.numpy().copy()
    slots[1] = nb * P + 3                       # out of range: skipped
    before = (_bits(x.cache) if cache_dtype == "bf16" else x.cache.numpy()).copy()
    cache = before.copy()
    q = oracle.concat_insert(_bits(x.ql_nope), _bits(x.q_pe), _bits(x.kv_c), _bits(x.k_pe),
                             slots, cache, x.cache_scale_inv)
    # query: the two inputs side by side
    assert (q[:, :, :512] == _bits(x.ql_nope)).all() and (q[:, :, 512:] == _bits(x.q_pe)).all()
    row = np.concatenate([_bits(x.kv_c), _bits(x.k_pe)], axis=1)
    touched = np.zeros((nb, P), dtype=bool)
    for t, s in enumerate(slots):
        if s < 0 or s >= nb * P:
            continue
        blk, r = divmod(int(s), P)
        touched[blk, r] = True
        if cache_dtype == "bf16":
            assert (cache[blk, r] == row[t]).all()
        else:
            x_t = np.array([oracle.bf16_to_double(int(b)) for b in row[t]])
            back = np.array([oracle.e4m3fn_to_double(int(c)) for c in cache[blk, r]])
            scale = 1.0 / x.cache_scale_inv
            # within half a code step: relative 2^-4 for normals, 2^-10 absolute
            # (times the scale) in the subnormal range
            err = np.abs(back * scale - x_t)
            tol = np.maximum(np.abs(x_t) * 2.0 ** -4, 2.0 ** -10 * scale) * 1.001
            assert (err <= tol).all(), float((err / tol).max())
    assert (cache[~touched] == before[~touched]).all()
    assert touched.sum() == ((slots >= 0) & (slots < nb * P)).sum()
