"""Multi-token decode (uniform query length, causal or not) through the C ABI
against the oracle, on every split kernel (N = 16, 64, 128; bf16 and fp8),
several split counts, and requests shorter than q_len."""
import numpy as np
import pytest
import torch

import oracle
from head_latent_attention_decode_amd import mla
from head_latent_attention_decode_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _run_and_check(wl, QL, S, causal, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(wl.B, QL, wl.N, 576, generator=g).to(torch.bfloat16)
    d = G.to_device(wl)
    out, lse = mla.mla_decode_multi(q.cuda(), d["latent_cache"], d["block_table"],
                                    d["seq_lens"], wl.softmax_scale, S, causal=causal,
                                    cache_scale=d["cache_scale"], cache_dtype=d["cache_dtype"])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.mla_decode_multi(q.double().numpy(), wl.cache_bits(),
                                           wl.block_table.numpy(), wl.seq_lens.numpy(),
                                           wl.softmax_scale, QL, causal=causal,
                                           cache_scale=wl.cache_scale)
    lens = np.repeat(wl.seq_lens.numpy()[:, None], QL, axis=1).astype(np.int64)
    if causal:
        lens = lens - (QL - 1 - np.arange(QL)[None, :])
    lens = np.maximum(lens, 0)
    row_lens = np.repeat(lens[:, :, None], wl.N, axis=2)
    G.check(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, row_lens,
            dtype=wl.cache_dtype, what=f"QL={QL} S={S} causal={causal}")


@pytest.mark.parametrize("N,cache_dtype", [(16, "bf16"), (64, "bf16"), (128, "bf16"),
                                           (128, "fp8_e4m3fn")])
@pytest.mark.parametrize("QL,S,causal", [(2, 1, True), (4, 3, True), (8, 2, False),
                                         (3, 1, False)])
def test_multi_token_decode_matches_oracle(N, cache_dtype, QL, S, causal):
    wl = W.make_workload(4, N, 16, [1, 5, 300, 1100], seed=N + QL, cache_dtype=cache_dtype)
    _run_and_check(wl, QL, S, causal, seed=QL * 31 + S)


def test_multi_token_rejects_bad_q_len():
    wl = W.make_workload(1, 16, 16, [10], seed=1)
    d = G.to_device(wl)
    q = torch.zeros(1, 17, 16, 576, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MLAError):
        mla.mla_decode_multi(q, d["latent_cache"], d["block_table"], d["seq_lens"],
                             wl.softmax_scale, 1)


@pytest.mark.parametrize("QL", [4, 8])
@pytest.mark.parametrize("S", [1, 2])
@pytest.mark.parametrize("causal", [True, False])
def test_multi_token_rows_share_a_workgroup(QL, S, causal):
    """N = 16 with q_len 4 or 8: a workgroup holds 64 heads of several query
    rows, each masked at its own causal end.  L = 2049 at S = 2 leaves a
    one-token last chunk in which the earlier causal rows have no token, and
    L = 2 < q_len leaves whole rows empty."""
    wl = W.make_workload(4, 16, 64, [2, 2049, 4100, 33], seed=70 + QL + S, max_len=4160)
    _run_and_check(wl, QL, S, causal, seed=QL * 7 + S + int(causal))
