"""Concurrent calls on two streams (needs an MI355X).

The library keeps no state between calls (mla_decode_noalloc aside), so
decodes of different batches with their own workspaces and outputs may run
at the same time on different streams.  Calls are launched alternately on
two default-priority streams, so that their kernels overlap on the device,
and every result is compared bit for bit with the same call made alone.
"""
import pytest
import torch

from head_latent_attention_decode_amd import mla
from head_latent_attention_decode_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _call(d, wl, S, out, lse, ws):
    return mla.mla_decode(d["q"], d["latent_cache"], d["block_table"], d["seq_lens"],
                          wl.softmax_scale, S, out=out, lse=lse, workspace=ws,
                          cache_scale=d["cache_scale"], cache_dtype=d["cache_dtype"])


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8_e4m3fn"])
def test_two_streams_match_serial(cache_dtype):
    cases = []
    for k, (N, S, lens) in enumerate([(128, 8, [3000, 17, 9000, 4096, 1]),
                                      (16, 16, [20000, 513, 7]),
                                      (64, 2, [2049, 100, 6000, 32, 1000, 5]),
                                      (128, 1, [700, 64, 3333])]):
        wl = W.make_workload(len(lens), N, 64, lens, seed=1300 + k, cache_dtype=cache_dtype)
        d = G.to_device(wl)
        shape = mla.make_shape(d["q"], d["latent_cache"], d["block_table"], d["cache_dtype"])
        ws = torch.empty(max(1, mla.workspace_size(shape, S)), dtype=torch.uint8, device="cuda")
        out = torch.empty((wl.B, N, W.KV_LORA_RANK), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((wl.B, N), dtype=torch.float32, device="cuda")
        cases.append((wl, d, S, out, lse, ws))

    # each call alone
    ref = []
    for wl, d, S, out, lse, ws in cases:
        _call(d, wl, S, out, lse, ws)
        torch.cuda.synchronize()
        ref.append((out.clone(), lse.clone()))

    # the same calls, alternating between two streams, several rounds
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rnd in range(3):
        for _, _, _, out, lse, _ in cases:
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
        torch.cuda.synchronize()
        for i, (wl, d, S, out, lse, ws) in enumerate(cases):
            with torch.cuda.stream(streams[i % 2]):
                _call(d, wl, S, out, lse, ws)
        torch.cuda.synchronize()
        for i, ((_, _, _, out, lse, _), (ro, rl)) in enumerate(zip(cases, ref)):
            print(f"{cache_dtype} round {rnd} case {i}", flush=True)
            assert torch.equal(_bits(out), _bits(ro)), f"round {rnd} case {i}: out differs"
            assert torch.equal(_bits(lse), _bits(rl)), f"round {rnd} case {i}: lse differs"
