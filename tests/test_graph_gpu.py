"""HIP-graph capture of the decode step (needs an MI355X).

A serving loop records one decode step into a graph once and replays it with
each step's inputs written into the same buffers.  The library allocates
nothing and issues no memset, so a captured mla_decode (split kernel, then
the merge) or mla_decode_noalloc is a plain chain of kernel nodes, and the
lengths are read from device memory at run time, so one graph serves any
lengths within the page table's capacity.

Each replay is compared bit for bit with an eager call on the same inputs;
the inputs change between replays (new query, cache contents, page table and
per-request lengths), and eager work and synchronisations run between the
replays.
"""
import pytest
import torch

from head_latent_attention_decode_amd import mla
from head_latent_attention_decode_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

LENS = [1, 100, 2049, 5000, 7777, 333]
REPLAYS = 4


def _say(*a):
    print(*a, flush=True)


def _workload(N, cache_dtype, r):
    # the same multiset of lengths, rotated: identical tensor shapes, other
    # per-request lengths, contents and page placement
    lens = LENS[r % len(LENS):] + LENS[:r % len(LENS)]
    return W.make_workload(len(lens), N, 64, lens, seed=900 + 17 * r + N,
                           cache_dtype=cache_dtype)


def _load_into(bufs, wl):
    d = G.to_device(wl)
    for k in ("q", "latent_cache", "block_table", "seq_lens"):
        assert bufs[k].shape == d[k].shape and bufs[k].dtype == d[k].dtype
        bufs[k].copy_(d[k])
    if d["cache_scale"] is not None:
        bufs["cache_scale"].copy_(d["cache_scale"])


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 \
        else torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("N,S,cache_dtype,noalloc", [
    (128, 4, "bf16", False),          # role-split kernel + merge
    (16, 8, "bf16", False),           # 16-head kernel + merge
    (128, 4, "fp8_e4m3fn", False),
    (128, 1, "bf16", False),          # one split: the direct path, no merge
    (128, 4, "bf16", True),           # the allocation-free entry point
])
def test_graph_replay_matches_eager(N, S, cache_dtype, noalloc):
    wl0 = _workload(N, cache_dtype, 0)
    bufs = G.to_device(wl0)
    scale = wl0.softmax_scale
    B = wl0.B
    dev = bufs["q"].device
    out_g = torch.empty((B, N, W.KV_LORA_RANK), dtype=torch.bfloat16, device=dev)
    lse_g = torch.empty((B, N), dtype=torch.float32, device=dev)
    shape = mla.make_shape(bufs["q"], bufs["latent_cache"], bufs["block_table"],
                           bufs["cache_dtype"])
    ws = torch.empty(max(1, mla.workspace_size(shape, S)), dtype=torch.uint8, device=dev)

    def step(out, lse, workspace):
        if noalloc:
            return mla.mla_decode_noalloc(bufs["q"], bufs["latent_cache"], bufs["block_table"],
                                          bufs["seq_lens"], scale, S, out=out, lse=lse,
                                          cache_scale=bufs["cache_scale"],
                                          cache_dtype=bufs["cache_dtype"])
        return mla.mla_decode(bufs["q"], bufs["latent_cache"], bufs["block_table"],
                              bufs["seq_lens"], scale, S, out=out, lse=lse,
                              workspace=workspace, cache_scale=bufs["cache_scale"],
                              cache_dtype=bufs["cache_dtype"])

    # warm up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out_g, lse_g, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_g, lse_g, ws)
    torch.cuda.synchronize()

    out_e = torch.empty_like(out_g)
    lse_e = torch.empty_like(lse_g)
    ws_e = torch.empty_like(ws)
    for r in range(REPLAYS):
        _load_into(bufs, _workload(N, cache_dtype, r))
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        # eager work between the replay and the reference call
        junk = torch.randn(1 << 20, device=dev).sum()
        step(out_e, lse_e, ws_e)
        torch.cuda.synchronize()
        _say(f"N={N} S={S} {cache_dtype} noalloc={noalloc} replay {r}: junk {float(junk):.3f}")
        assert _same(out_g, out_e), f"replay {r}: out differs from the eager call"
        assert _same(lse_g, lse_e), f"replay {r}: lse differs from the eager call"

    # the last replay's inputs, checked against the oracle too
    wl = _workload(N, cache_dtype, REPLAYS - 1)
    ref_o, ref_l = G.reference(wl)
    G.check(out_g.float().cpu(), lse_g.cpu(), ref_o, ref_l, G.row_lens(wl), dtype=cache_dtype,
            what=f"graph N={N} S={S} {cache_dtype}")
