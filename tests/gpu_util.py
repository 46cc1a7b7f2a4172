"""Shared helpers of the GPU tests: device transfer, runs through the C ABI,
oracle references and the tolerance checks."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from head_latent_attention_decode_amd import mla

# Tolerances (max relative error of a row's output in the infinity norm, max
# absolute error of the natural-log LSE): bf16 cache 1e-2 / 2e-3; fp8 cache
# 5e-2 on both.
TOL = {"bf16": (1e-2, 2e-3), "fp8_e4m3fn": (5e-2, 5e-2)}


def to_device(wl, dev="cuda"):
    d = dict(q=wl.q.to(dev), latent_cache=wl.cache.to(dev),
             block_table=wl.block_table.to(dev), seq_lens=wl.seq_lens.to(dev))
    d["cache_scale"] = (torch.tensor([wl.cache_scale], dtype=torch.float32, device=dev)
                        if wl.cache_dtype == "fp8_e4m3fn" else None)
    d["cache_dtype"] = wl.cache_dtype
    return d


def run(wl, S=None, dev_inputs=None, **kw):
    """mla_decode through the C ABI; returns (out float32 CPU, lse float32 CPU)."""
    d = dev_inputs or to_device(wl)
    out, lse = mla.mla_decode(d["q"], d["latent_cache"], d["block_table"], d["seq_lens"],
                              wl.softmax_scale, S or wl.num_kv_splits,
                              cache_scale=d["cache_scale"], cache_dtype=d["cache_dtype"], **kw)
    torch.cuda.synchronize()
    return out.float().cpu(), (lse.cpu() if lse is not None else None)


def problem(wl):
    return oracle.Problem(wl.q_float64(), wl.cache_bits(), wl.block_table.numpy(),
                          wl.seq_lens.numpy(), wl.softmax_scale, cache_scale=wl.cache_scale)


def reference(wl, rows=None):
    return oracle.mla_decode(problem(wl), rows=rows)


def reference_all_rows(wl, requests_per_call=8, say=print):
    """The oracle on every (b, n) row of a workload, a few requests per call
    (all their heads), printing progress after each call so that a long run
    keeps reporting."""
    prob = problem(wl)
    B, N = wl.B, wl.N
    out = np.empty((B, N, prob.Dv))
    lse = np.empty((B, N))
    for b0 in range(0, B, requests_per_call):
        bs = np.arange(b0, min(B, b0 + requests_per_call))
        rb = np.repeat(bs, N)
        rn = np.tile(np.arange(N), len(bs))
        o, l = oracle.mla_decode(prob, rows=(rb, rn))
        out[bs] = o.reshape(len(bs), N, -1)
        lse[bs] = l.reshape(len(bs), N)
        say(f"  oracle rows of requests {b0}..{bs[-1]} of {B} done")
    return out, lse


def check(out, lse, ref_out, ref_lse, lens, dtype="bf16", what=""):
    """out/lse [..., Dv]/[...] from the GPU against the oracle; lens per row."""
    tol_o, tol_l = TOL[dtype]
    out = np.asarray(out, dtype=np.float64).reshape(-1, ref_out.shape[-1])
    ref_out = np.asarray(ref_out).reshape(-1, ref_out.shape[-1])
    lse = np.asarray(lse, dtype=np.float64).reshape(-1)
    ref_lse = np.asarray(ref_lse).reshape(-1)
    lens = np.asarray(lens).reshape(-1)
    empty = lens == 0
    assert (out[empty] == 0).all(), f"{what}: empty rows must be exactly 0"
    assert np.isneginf(lse[empty]).all(), f"{what}: empty rows must have lse = -inf"
    live = ~empty
    if not live.any():
        return 0.0, 0.0
    assert np.isfinite(out[live]).all() and np.isfinite(lse[live]).all(), f"{what}: non-finite"
    err = np.abs(out[live] - ref_out[live]).max(axis=1) / np.abs(ref_out[live]).max(axis=1)
    lerr = np.abs(lse[live] - ref_lse[live])
    assert err.max() <= tol_o, f"{what}: out rel err {err.max():.3e} > {tol_o}"
    assert lerr.max() <= tol_l, f"{what}: lse abs err {lerr.max():.3e} > {tol_l}"
    return float(err.max()), float(lerr.max())


def row_lens(wl):
    """KV length of every (b, n) row."""
    return np.repeat(wl.seq_lens.numpy()[:, None], wl.N, axis=1)
