"""The per-head matmuls around the attention (query absorb with W_UK_T, output
up-projection with W_UV) through the C ABI against the oracle's fp64
absorb_query / up_project (pinned by the MHA == absorbed-MQA identity).  The
weights are prepared in the pages' layouts: W_UK_T = W_UK.permute(1, 2, 0),
W_UV.transpose(0, 1)."""
import numpy as np
import pytest
import torch

from head_latent_attention_decode_amd import mla
from head_latent_attention_decode_amd import workloads as W
from oracle import mha

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _rel_rows(got, ref):
    got = got.reshape(-1, got.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    return (np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)).max()


@pytest.mark.parametrize("B,N", [(1, 16), (37, 16), (64, 128), (256, 128), (5, 8), (100, 24), (3, 3), (300, 16)])
def test_absorb_and_up_project_match_oracle(B, N):
    x = W.make_projection_inputs(B, N, seed=B * 3 + N)
    w_uk_t = x.W_UK.permute(1, 2, 0).contiguous().to(DEV)
    w_uv = x.W_UV.transpose(0, 1).contiguous().to(DEV)
    ql = mla.absorb_query(x.q_nope.to(DEV), w_uk_t)
    up = mla.up_project(x.latent_out.to(DEV), w_uv)
    torch.cuda.synchronize()
    WUK, WUV = x.W_UK.double().numpy(), x.W_UV.double().numpy()
    qn, lat = x.q_nope.double().numpy(), x.latent_out.double().numpy()
    ref_ql = np.stack([mha.absorb_query(qn[b], np.zeros((N, 64)), WUK)[:, :512] for b in range(B)])
    ref_up = np.stack([mha.up_project(lat[b], WUV) for b in range(B)])
    assert _rel_rows(ql.float().cpu().numpy(), ref_ql) <= 8e-3
    assert _rel_rows(up.float().cpu().numpy(), ref_up) <= 8e-3


def test_absorb_reads_a_strided_slice():
    """q_nope as the first 128 columns of a [B, N, 192] query (nope + rope)."""
    B, N = 19, 16
    x = W.make_projection_inputs(B, N, seed=5)
    full = torch.zeros(B, N, 192, dtype=torch.bfloat16)
    full[..., :128] = x.q_nope
    full[..., 128:] = float("nan")                 # never read
    w_uk_t = x.W_UK.permute(1, 2, 0).contiguous().to(DEV)
    ql = mla.absorb_query(full.to(DEV)[..., :128], w_uk_t)
    ref = mla.absorb_query(x.q_nope.to(DEV), w_uk_t)
    torch.cuda.synchronize()
    assert torch.equal(ql, ref)
