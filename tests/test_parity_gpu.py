"""Parity of the HIP decode path with the fp64 oracle (needs an MI355X).

Every call goes through the C ABI (libmla_decode.so) via the ctypes binding.
Every case, the five named workloads at full size included, is compared with
the oracle on every (b, n) row, element by element.
"""
import numpy as np
import pytest
import torch

import oracle
from head_latent_attention_decode_amd import mla
from head_latent_attention_decode_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

LENS = [1, 17, 31, 32, 33, 100, 129, 1000]


def _say(*a):
    print(*a, flush=True)


def test_tiny_workload():
    wl = W.config_workload("tiny")
    out, lse = G.run(wl)
    ref_o, ref_l = G.reference(wl)
    e = G.check(out, lse, ref_o, ref_l, G.row_lens(wl), what="tiny")
    _say("tiny", e)


@pytest.mark.parametrize("N", [16, 32, 48, 128, 256])
@pytest.mark.parametrize("page", [16, 64])
@pytest.mark.parametrize("S", [1, 3, 8])
def test_small_grid(N, page, S):
    wl = W.make_workload(len(LENS), N, page, LENS, seed=100 + N + page + S)
    _say("case", N, page, S)
    out, lse = G.run(wl, S)
    ref_o, ref_l = G.reference(wl)
    G.check(out, lse, ref_o, ref_l, G.row_lens(wl), what=f"N={N} P={page} S={S}")


@pytest.mark.parametrize("N", [16, 64, 128])
@pytest.mark.parametrize("page", [16, 64])
@pytest.mark.parametrize("S", [1, 2, 5])
def test_fp8_small(N, page, S):
    # 2100 tokens at 16-token pages cross the 64-page window of the tile loader
    lens = [1, 40, 64, 65, 300, 777, 2100]
    wl = W.make_workload(len(lens), N, page, lens, seed=200 + N + page + S,
                         cache_dtype="fp8_e4m3fn")
    _say("fp8 case", N, page, S)
    out, lse = G.run(wl, S)
    ref_o, ref_l = G.reference(wl)
    G.check(out, lse, ref_o, ref_l, G.row_lens(wl), dtype="fp8_e4m3fn", what=f"fp8 N={N} P={page} S={S}")


@pytest.mark.parametrize("N", [64, 128])
@pytest.mark.parametrize("page", [16, 64])
@pytest.mark.parametrize("S", [2, 3])
def test_fp8_chunks_off_the_tile_grid(N, page, S):
    """fp8 tiles are 64 tokens while chunk lengths are multiples of 32, so a
    chunk may start half-way through a 64-token block and end in a 32-token
    tile: 4160 and 4100 tokens at S = 2 give chunks of 2080, and 6600 at
    S = 3 chunks of 2208."""
    lens = [4160, 4100, 6600, 2081, 33]
    wl = W.make_workload(len(lens), N, page, lens, seed=1100 + N + page + S,
                         cache_dtype="fp8_e4m3fn")
    _say("fp8 off-grid", N, page, S)
    out, lse = G.run(wl, S)
    ref_o, ref_l = G.reference(wl)
    G.check(out, lse, ref_o, ref_l, G.row_lens(wl), dtype="fp8_e4m3fn",
            what=f"fp8 off-grid N={N} P={page} S={S}")


@pytest.mark.parametrize("page", [32, 128, 256, 1024])
@pytest.mark.parametrize("N,cache_dtype", [(16, "bf16"), (128, "bf16"), (16, "fp8_e4m3fn"),
                                           (128, "fp8_e4m3fn")])
def test_other_page_sizes(page, N, cache_dtype):
    """Power-of-two page sizes the boundary accepts besides the configs' 16
    and 64, up to its largest, 1024: lengths on both sides of a page end, and
    at page 32 a request (5000 tokens) past the 64-page window of the
    page-table reads."""
    lens = [1, 100, 1023, 1024, 1025, 5000]
    wl = W.make_workload(len(lens), N, page, lens, seed=1000 + page + N,
                         cache_dtype=cache_dtype)
    ref_o, ref_l = G.reference(wl)
    for S in (1, 3):
        _say("page", page, N, cache_dtype, S)
        out, lse = G.run(wl, S)
        G.check(out, lse, ref_o, ref_l, G.row_lens(wl), dtype=cache_dtype,
                what=f"P={page} N={N} {cache_dtype} S={S}")


@pytest.mark.parametrize("N", [16, 128])
@pytest.mark.parametrize("S", [1, 4])
def test_zero_length_rows(N, S):
    lens = [0, 5, 0, 70]
    wl = W.make_workload(4, N, 16, lens, seed=300 + N, max_len=128)
    out, lse = G.run(wl, S)
    ref_o, ref_l = G.reference(wl)
    G.check(out, lse, ref_o, ref_l, G.row_lens(wl), what=f"zero rows N={N} S={S}")


def test_all_rows_empty():
    wl = W.make_workload(3, 128, 64, [0, 0, 0], seed=7, max_len=64)
    for S in (1, 2):
        out, lse = G.run(wl, S)
        assert (out == 0).all() and torch.isneginf(lse).all()


@pytest.mark.parametrize("N", [16, 128])
def test_split_count_invariance(N):
    """out and lse do not depend on num_kv_splits (Model-Optimizer docs,
    mla_attention_decode, "Parameters", num_kv_splits): each S is compared
    with the oracle element by element, and with S = 1.  The 70000-token
    request is cut into 2, 3, 4, 7, 8, 32 and 35 live chunks by S = 2, 3, 4,
    7, 8, 32 and 64 (chunks of at least 2048 tokens), at boundaries that
    differ from one S to the next; the 20000-token one into 2 .. 10."""
    lens = [70000, 20000, 2049, 517, 64, 1]
    wl = W.make_workload(len(lens), N, 64, lens, seed=400 + N)
    _say("oracle", N)
    ref_o, ref_l = G.reference(wl)
    outs = {}
    for S in (1, 2, 3, 4, 7, 8, 32, 64):
        C = max(32 * -(-(-(-lens[0] // S)) // 32), 2048)
        _say("S", S, "live chunks of the longest request:", -(-lens[0] // C))
        out, lse = G.run(wl, S)
        G.check(out, lse, ref_o, ref_l, G.row_lens(wl), what=f"S={S}")
        outs[S] = (out, lse)
    # all split counts agree with each other to the same tolerance
    for S, (o, l) in outs.items():
        d = (o - outs[1][0]).abs().amax(-1) / outs[1][0].abs().amax(-1)
        assert float(d.max()) <= 1e-2, S
        assert float((l - outs[1][1]).abs().max()) <= 2e-3, S


@pytest.mark.parametrize("N", [16, 128])
def test_page_permutation_bitwise(N):
    lens = [300, 1, 129]
    a = W.make_workload(3, N, 16, lens, seed=500, perm_seed=1)
    b = W.make_workload(3, N, 16, lens, seed=500, perm_seed=2)
    assert not torch.equal(a.block_table, b.block_table)
    for S in (1, 3):
        oa, la = G.run(a, S)
        ob, lb = G.run(b, S)
        assert torch.equal(oa, ob) and torch.equal(la, lb), "result depends on page placement"


@pytest.mark.parametrize("N", [16, 128])
def test_run_to_run_bitwise(N):
    wl = W.make_workload(4, N, 64, [100, 2000, 5, 999], seed=600 + N)
    d = G.to_device(wl)
    first = G.run(wl, 4, dev_inputs=d)
    for _ in range(3):
        again = G.run(wl, 4, dev_inputs=d)
        assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])


@pytest.mark.parametrize("N", [16, 128])
@pytest.mark.parametrize("S", [8, 32])
def test_batch_invariance(N, S):
    """A request alone and the same request inside a batch give the same bits
    (at S = 32 the chunks of a request land on XCDs that depend on its index
    in the batch)."""
    lens = [700, 3000, 41] if S == 8 else [700, 70000, 41]
    big = W.make_workload(3, N, 64, lens, seed=700 + N)
    ob, lb = G.run(big, S)
    for b in range(3):
        L = int(lens[b])
        pages = -(-L // 64)
        one = W.Workload(name="one", q=big.q[b:b + 1].clone(), cache=big.cache,
                         block_table=big.block_table[b:b + 1, :pages].clone().contiguous(),
                         seq_lens=big.seq_lens[b:b + 1].clone(), softmax_scale=big.softmax_scale,
                         cache_scale=big.cache_scale, cache_dtype=big.cache_dtype,
                         num_kv_splits=S, seed=0)
        o1, l1 = G.run(one, S)
        assert torch.equal(o1[0], ob[b]) and torch.equal(l1[0], lb[b]), f"request {b}"


def test_no_lse_output():
    wl = W.make_workload(2, 128, 64, [90, 10], seed=800)
    out_a, _ = G.run(wl, 2)
    out_b, lse_b = G.run(wl, 2, return_lse=False)
    assert lse_b is None and torch.equal(out_a, out_b)


@pytest.mark.parametrize("N,S", [(16, 3), (128, 5)])
def test_partials_match_oracle_spans(N, S):
    """The split stage alone against the oracle's attention over each chunk,
    with chunk s = [s*C, min((s+1)*C, L)), C = max(32*ceil(ceil(L/S)/32), 2048).
    An empty chunk has lse = -inf; its output rows are unspecified."""
    lens = [1, 70, 5500, 64]
    wl = W.make_workload(4, N, 16, lens, seed=900 + N)
    d = G.to_device(wl)
    po, pl = mla.mla_decode_partials(d["q"], d["latent_cache"], d["block_table"], d["seq_lens"],
                                     wl.softmax_scale, S)
    torch.cuda.synchronize()
    po, pl = po.cpu().numpy(), pl.cpu().numpy()
    rb, rn, t0, t1 = [], [], [], []
    for b, L in enumerate(lens):
        C = max(32 * (-(-(-(-L // S)) // 32)), 2048)
        for n in range(N):
            for s in range(S):
                a = min(s * C, L)
                e = min(s * C + C, L)
                rb.append(b); rn.append(n); t0.append(a); t1.append(e)
    ref_o, ref_l = oracle.attend_spans(G.problem(wl), rb, rn, t0, t1)
    span = np.array(t1) - np.array(t0)
    po = po.reshape(-1, 512)
    po[span == 0] = 0.0                      # unspecified for an empty chunk
    # empty, whole and partial chunks all occur
    assert (span == 0).any() and (span == 2048).any() and ((span > 0) & (span < 2048)).any()
    G.check(po, pl.reshape(-1), ref_o, ref_l, span, what="partials")


@pytest.mark.parametrize("R,S", [(300, 7), (300, 9), (64, 64), (5000, 9)])
def test_merge_kernel_against_oracle(R, S):
    """One wave per row (few states, or many rows) and one workgroup per row
    (few rows with many states) against the oracle's merge."""
    g = torch.Generator().manual_seed(11 + S)
    po = torch.randn(R, S, 512, generator=g)
    pl = torch.randn(R, S, generator=g) * 3
    pl[torch.rand(R, S, generator=g) < 0.3] = -float("inf")
    pl[:5] = -float("inf")                       # rows with no weight at all
    po[torch.isneginf(pl)] = float("nan")        # never read: weight zero
    out, lse = mla.mla_merge_states(po.cuda(), pl.cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge_states(torch.nan_to_num(po).double().numpy(),
                                       pl.double().numpy())
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    assert (out[:5] == 0).all() and np.isneginf(lse[:5]).all()
    live = np.isfinite(ref_l)
    assert (np.isfinite(lse) == live).all()
    err = np.abs(out[live] - ref_o[live]).max(axis=1) / np.abs(ref_o[live]).max(axis=1)
    assert err.max() <= 8e-3, err.max()       # bf16 output rounding dominates
    assert np.abs(lse[live] - ref_l[live]).max() <= 1e-5


@pytest.mark.parametrize("name", ["dsv3", "ragged", "long_context", "fp8_cache"])
def test_full_size_workloads(name):
    """Each named workload at full size, in the launch configuration the
    benchmark times, against the oracle on every (b, n) row."""
    _say("generating", name)
    wl = W.config_workload(name)
    _say("running", name, "S =", wl.num_kv_splits)
    out, lse = G.run(wl)
    _say("oracle on all", wl.B * wl.N, "rows")
    ref_o, ref_l = G.reference_all_rows(wl, requests_per_call=8 if wl.N == 128 else 1, say=_say)
    e = G.check(out, lse, ref_o, ref_l, G.row_lens(wl), dtype=wl.cache_dtype, what=name)
    _say(name, "max errors (out rel, lse abs)", e)


@pytest.mark.parametrize("S", [8, 32])
def test_batch_invariance_across_merge_widths(S):
    """The merge's launch follows the row count (lanes own 8, 4, 2 or 1
    columns), its arithmetic does not: a request alone (128 rows) and inside a
    40-request batch (5120 rows) gives the same bits."""
    rng = np.random.default_rng(S)
    lens = [int(x) for x in rng.integers(1, 20000, size=40)]
    lens[0], lens[1] = 19999, 2049
    big = W.make_workload(40, 128, 64, lens, seed=1200 + S)
    ob, lb = G.run(big, S)
    for b in (0, 1, 7):
        pages = -(-lens[b] // 64)
        one = W.Workload(name="one", q=big.q[b:b + 1].clone(), cache=big.cache,
                         block_table=big.block_table[b:b + 1, :pages].clone().contiguous(),
                         seq_lens=big.seq_lens[b:b + 1].clone(), softmax_scale=big.softmax_scale,
                         cache_scale=big.cache_scale, cache_dtype=big.cache_dtype,
                         num_kv_splits=S, seed=0)
        o1, l1 = G.run(one, S)
        assert torch.equal(o1[0], ob[b]) and torch.equal(l1[0], lb[b]), f"request {b}"


def test_merge_bits_do_not_depend_on_row_count():
    """Rows 0..4 merged alone, and among 200, 1000 and 5000 rows (each launch
    width of the merge), give the same bits."""
    g = torch.Generator().manual_seed(5)
    S = 40
    po = torch.randn(5000, S, 512, generator=g)
    pl = torch.randn(5000, S, generator=g) * 4
    pl[torch.rand(5000, S, generator=g) < 0.4] = -float("inf")
    pl[3] = -float("inf")
    po_d, pl_d = po.cuda(), pl.cuda()
    first = None
    for R in (5, 200, 1000, 5000):
        out, lse = mla.mla_merge_states(po_d[:R].contiguous(), pl_d[:R].contiguous())
        torch.cuda.synchronize()
        got = (out[:5].cpu(), lse[:5].cpu())
        if first is None:
            first = got
        assert torch.equal(got[0], first[0]) and torch.equal(got[1], first[1]), R
    assert (first[0][3] == 0).all() and torch.isneginf(first[1][3])


def test_binding_refuses_bad_lengths_and_outputs():
    """seq_lens must hold B entries and caller outputs must match the call:
    the binding raises before the library could read or write out of
    bounds."""
    wl = W.make_workload(2, 16, 16, [30, 5], seed=9)
    d = G.to_device(wl)
    args = (d["q"], d["latent_cache"], d["block_table"])
    with pytest.raises(ValueError):
        mla.mla_decode(*args, d["seq_lens"][:1], wl.softmax_scale, 2)
    with pytest.raises(ValueError):
        mla.mla_decode(*args, d["seq_lens"], wl.softmax_scale, 2,
                       out=torch.empty((2, 16, 256), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        mla.mla_decode(*args, d["seq_lens"], wl.softmax_scale, 2,
                       lse=torch.empty((2, 8), dtype=torch.float32, device="cuda"))
