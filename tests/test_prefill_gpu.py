"""Chunked-context gather and two-state merge on the GPU against the oracle:
bit-exact gather rows (a copy, or for fp8 a bf16 value decided in fp32 on
both sides) and the merge within bf16 output rounding, also in place."""
import numpy as np
import pytest
import torch

import oracle
from head_latent_attention_decode_amd import mla
from head_latent_attention_decode_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("cache_dtype,align,P", [("bf16", True, 16), ("bf16", False, 64),
                                                 ("fp8_e4m3fn", True, 64),
                                                 ("fp8_e4m3fn", False, 16)])
def test_gather_matches_oracle_bitwise(cache_dtype, align, P):
    wl = W.make_workload(5, 16, P, [1, 300, 77, 1024, 513], seed=31, cache_dtype=cache_dtype)
    g = W.make_gather_inputs(wl, seed=9, chunk_tokens=400, align=align)
    cache_np = _bits(wl.cache) if cache_dtype == "bf16" else wl.cache.numpy()
    ref = oracle.gather(cache_np, g.block_table.numpy(), g.cu_seq_lens.numpy(),
                        g.token_to_seq.numpy(), g.seq_starts.numpy(), scale=wl.cache_scale)
    scale = torch.tensor([wl.cache_scale], dtype=torch.float32, device=DEV)
    got = mla.gather_cache(wl.cache.to(DEV), g.block_table.to(DEV), g.cu_seq_lens.to(DEV),
                           g.token_to_seq.to(DEV), seq_starts=g.seq_starts.to(DEV),
                           cache_scale=scale if cache_dtype != "bf16" else None,
                           cache_dtype=cache_dtype)
    torch.cuda.synchronize()
    assert got.shape == (int(g.cu_seq_lens[-1]), 576)
    assert (_bits(got) == ref).all(), int((_bits(got) != ref).sum())


def test_gather_without_starts_reads_from_token_zero():
    wl = W.make_workload(2, 16, 16, [50, 20], seed=2)
    cu = torch.tensor([0, 50, 70], dtype=torch.int32)
    tts = torch.tensor([0] * 50 + [1] * 20, dtype=torch.int32)
    ref = oracle.gather(_bits(wl.cache), wl.block_table.numpy(), cu.numpy(), tts.numpy())
    got = mla.gather_cache(wl.cache.to(DEV), wl.block_table.to(DEV), cu.to(DEV), tts.to(DEV))
    torch.cuda.synchronize()
    assert (_bits(got) == ref).all()


def _check_merge(m, out, lse):
    ref_o, ref_l = oracle.merge_two(m.prefix_out.double().numpy(), m.prefix_lse.double().numpy(),
                                    m.suffix_out.double().numpy(), m.suffix_lse.double().numpy())
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    T, N, D = out.shape
    o2, r2 = out.reshape(-1, D), ref_o.reshape(-1, D)
    live = np.isfinite(ref_l.T.reshape(-1))
    assert (o2[~live] == 0).all() and np.isneginf(lse.T.reshape(-1)[~live]).all()
    if not live.any():
        return
    err = np.abs(o2[live] - r2[live]).max(axis=1) / np.abs(r2[live]).max(axis=1)
    assert err.max() <= 8e-3, err.max()          # bf16 output rounding dominates
    assert np.abs(lse.T.reshape(-1)[live] - ref_l.T.reshape(-1)[live]).max() <= 1e-5


@pytest.mark.parametrize("T,N,D", [(1, 1, 8), (37, 16, 128), (300, 128, 128), (64, 8, 512),
                                   (5, 3, 2048)])
def test_merge_attn_states_matches_oracle(T, N, D):
    m = W.make_merge_inputs(T, N, D, seed=T + N + D)
    out, lse = mla.merge_attn_states(m.prefix_out.to(DEV), m.prefix_lse.to(DEV),
                                     m.suffix_out.to(DEV), m.suffix_lse.to(DEV))
    torch.cuda.synchronize()
    _check_merge(m, out, lse)


def test_merge_attn_states_in_place():
    """Folding a suffix into the running prefix, output over the prefix."""
    m = W.make_merge_inputs(200, 16, 128, seed=77)
    po, pl = m.prefix_out.to(DEV), m.prefix_lse.to(DEV)
    out, lse = mla.merge_attn_states(po, pl, m.suffix_out.to(DEV), m.suffix_lse.to(DEV),
                                     out=po, out_lse=pl)
    torch.cuda.synchronize()
    assert out.data_ptr() == po.data_ptr() and lse.data_ptr() == pl.data_ptr()
    _check_merge(m, out, lse)
