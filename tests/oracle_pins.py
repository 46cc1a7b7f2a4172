"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with what the pages and the
mathematics fix.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on deliberately broken copies of the
oracle source and requires every copy to fail at least one of them.

What each pin rests on:
  * E4M3 / bf16 decoding: the library's own float8_e4m3fn / bfloat16
    conversions (torch), over every code.
  * one-token context: softmax of one score is 1, so out is the value row and
    the LSE is the score itself.
  * 1-3 token contexts: the softmax definition exp(s_t) / sum exp(s_j),
    written with math.fsum in plain Python, without the max shift.
  * q = 0: every score is 0, so lse = ln L and out is the column mean.
  * identical rows: out is the row, lse = s + ln L.
  * column roles: the value is the first 512 columns of a row (kv_c) and the
    last 64 (k_pe) only enter the scores (vLLM API docs module docstring,
    forward_mqa: SDPA(cat[ql_nope, q_pe], cat[kv_c, k_pe], kv_c)).
  * absorbed MQA == explicit MHA with per-head up-projection (the two
    formulations of the same docstring) on random weights.
  * split + LSE merge == unsplit for any boundaries; (0, -inf) is neutral.
  * permuting physical pages together with the page table changes no bit.
  * an fp8 cache with a power-of-two scale equals the bf16 cache holding the
    decoded, rescaled values, bit for bit.
  * hand-worked examples in tests/golden/.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import mha

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
D, DV = 576, 512


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _paged(rows_per_req, page_size, rng, dqk=D, poison_bits=0x7FC0, dtype=np.uint16):
    """Scatter each request's rows (raw bits [L, dqk]) into a shuffled paged
    cache whose other rows hold NaN; returns (cache, block_table, seq_lens)."""
    B = len(rows_per_req)
    lens = [r.shape[0] for r in rows_per_req]
    pages = [(L + page_size - 1) // page_size for L in lens]
    total = sum(pages)
    perm = rng.permutation(total)
    nb = total + 1
    cache = np.full((nb, page_size, dqk), poison_bits, dtype=dtype)
    mb = max(1, max(pages) if pages else 1)
    table = np.full((B, mb), total, dtype=np.int32)
    k = 0
    for b, rows in enumerate(rows_per_req):
        for i in range(pages[b]):
            table[b, i] = perm[k]
            seg = rows[i * page_size:(i + 1) * page_size]
            cache[perm[k], :seg.shape[0]] = seg
            k += 1
    return cache, table, np.array(lens, dtype=np.int32)


def _problem(q, rows_per_req, page_size=16, scale=0.125, rng=None, dv=DV):
    rng = rng or np.random.default_rng(0)
    cache, table, lens = _paged(rows_per_req, page_size, rng, dqk=q.shape[-1])
    return oracle.Problem(q, cache, table, lens, scale, dv=dv)


def _rand_rows(rng, L, dqk=D):
    return _bf16_bits(rng.standard_normal((L, dqk)).astype(np.float32))


def _rand_q(rng, B, N, dqk=D):
    return _bits_to_f64(_bf16_bits(rng.standard_normal((B, N, dqk)).astype(np.float32)))


# ---------------------------------------------------------------- decoding

def pin_e4m3_table(lib):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3fn_to_double(c, lib) for c in range(256)])
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert (nan_ref == nan_got).all(), "E4M3 NaN codes differ"
    assert (ref[~nan_ref] == got[~nan_got]).all(), "E4M3 decode differs from torch"
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def pin_bf16_decode(lib):
    rng = np.random.default_rng(1)
    bits = np.concatenate([rng.integers(0, 65536, 4000), [0x3F80, 0xBF80, 0x0001, 0x7F7F]])
    ref = _bits_to_f64(bits.astype(np.uint16))
    got = np.array([oracle.bf16_to_double(int(b), lib) for b in bits])
    fin = np.isfinite(ref)
    assert (ref[fin] == got[fin]).all(), "bf16 decode differs from torch"


# ---------------------------------------------------------------- closed forms

def pin_single_token(lib):
    rng = np.random.default_rng(2)
    q = _rand_q(rng, 3, 4)
    rows = [_rand_rows(rng, 1) for _ in range(3)]
    p = _problem(q, rows, page_size=16, scale=0.07, rng=rng)
    out, lse = oracle.mla_decode(p, lib=lib, nthreads=2)
    for b in range(3):
        K = _bits_to_f64(rows[b])[0]
        for n in range(4):
            s = float(np.float32(0.07)) * float(np.dot(q[b, n], K))
            assert abs(lse[b, n] - s) <= 1e-12 * max(1.0, abs(s)), (b, n, lse[b, n], s)
            assert (out[b, n] == K[:DV]).all(), "one-token output must be the value row"


def pin_brute_force_tiny(lib):
    rng = np.random.default_rng(3)
    q = _rand_q(rng, 3, 2)
    lens = [2, 3, 3]
    rows = [_rand_rows(rng, L) for L in lens]
    scale = float(np.float32(1 / math.sqrt(192)))
    # page size 2 puts the second and third tokens on different pages
    p = _problem(q, rows, page_size=2, scale=scale, rng=rng)
    out, lse = oracle.mla_decode(p, lib=lib, nthreads=1)
    for b, L in enumerate(lens):
        K = _bits_to_f64(rows[b]).tolist()
        for n in range(2):
            qv = q[b, n].tolist()
            s = [scale * math.fsum(qv[d] * K[t][d] for d in range(D)) for t in range(L)]
            e = [math.exp(x) for x in s]
            z = math.fsum(e)
            want_lse = math.log(z)
            assert abs(lse[b, n] - want_lse) < 1e-12, (lse[b, n], want_lse)
            for l in range(0, DV, 37):
                want = math.fsum(e[t] / z * K[t][l] for t in range(L))
                assert abs(out[b, n, l] - want) < 1e-12, (b, n, l)


def pin_zero_query(lib):
    rng = np.random.default_rng(4)
    lens = [1, 5, 33, 100]
    rows = [_rand_rows(rng, L) for L in lens]
    q = np.zeros((4, 2, D))
    p = _problem(q, rows, page_size=16, rng=rng)
    out, lse = oracle.mla_decode(p, lib=lib, nthreads=2)
    for b, L in enumerate(lens):
        mean = _bits_to_f64(rows[b])[:, :DV].mean(axis=0)
        for n in range(2):
            assert abs(lse[b, n] - math.log(L)) < 1e-14, "q = 0 must give lse = ln L"
            assert np.allclose(out[b, n], mean, rtol=0, atol=1e-13)


def pin_identical_rows(lib):
    rng = np.random.default_rng(5)
    row = _rand_rows(rng, 1)
    L = 77
    q = _rand_q(rng, 1, 3)
    p = _problem(q, [np.repeat(row, L, axis=0)], page_size=16, scale=0.1, rng=rng)
    out, lse = oracle.mla_decode(p, lib=lib, nthreads=1)
    K = _bits_to_f64(row)[0]
    for n in range(3):
        s = float(np.float32(0.1)) * float(np.dot(q[0, n], K))
        assert abs(lse[0, n] - (s + math.log(L))) < 1e-12
        assert np.allclose(out[0, n], K[:DV], rtol=1e-14, atol=0)


def pin_column_roles(lib):
    rng = np.random.default_rng(6)
    L = 40
    rows = _rand_rows(rng, L)
    q = _rand_q(rng, 1, 2)
    # (a) with q_pe = 0 the rope columns must not matter at all
    qa = q.copy()
    qa[..., DV:] = 0
    alt = rows.copy()
    alt[:, DV:] = _rand_rows(rng, L)[:, DV:]
    o1, l1 = oracle.mla_decode(_problem(qa, [rows], rng=np.random.default_rng(9)), lib=lib)
    o2, l2 = oracle.mla_decode(_problem(qa, [alt], rng=np.random.default_rng(9)), lib=lib)
    assert (o1 == o2).all() and (l1 == l2).all(), "k_pe columns leaked into out or were mis-scored"
    # (b) with q_nope = 0 the scores come only from the rope columns
    qb = q.copy()
    qb[..., :DV] = 0
    alt2 = rows.copy()
    alt2[:, :DV] = _rand_rows(rng, L)[:, :DV]
    _, l3 = oracle.mla_decode(_problem(qb, [rows], rng=np.random.default_rng(9)), lib=lib)
    _, l4 = oracle.mla_decode(_problem(qb, [alt2], rng=np.random.default_rng(9)), lib=lib)
    assert (l3 == l4).all(), "kv_c columns entered the rope-only scores"
    # (c) the rope columns do enter the scores when q_pe != 0
    _, l5 = oracle.mla_decode(_problem(q, [rows], rng=np.random.default_rng(9)), lib=lib)
    _, l6 = oracle.mla_decode(_problem(q, [alt], rng=np.random.default_rng(9)), lib=lib)
    assert (l5 != l6).any(), "k_pe columns were ignored in the scores"


def pin_mha_equals_absorbed(lib):
    """forward_mha (up-projected per head) == forward_mqa (absorbed) on random weights."""
    rng = np.random.default_rng(7)
    N, P, R, V, Lkv = 4, 128, 64, 128, DV
    Skv = 23
    rows = _rand_rows(rng, Skv)
    Kf = _bits_to_f64(rows)
    kv_c, k_pe = Kf[:, :Lkv], Kf[:, Lkv:]
    W_UK = rng.standard_normal((Lkv, N, P)) / math.sqrt(Lkv)
    W_UV = rng.standard_normal((Lkv, N, V)) / math.sqrt(Lkv)
    q_nope = rng.standard_normal((N, P))
    q_pe = rng.standard_normal((N, R))
    scale = float(np.float32(1 / math.sqrt(P + R)))
    o_mha, lse_mha = mha.mha_decode(q_nope, q_pe, kv_c, k_pe, W_UK, W_UV, scale)
    q_abs = mha.absorb_query(q_nope, q_pe, W_UK)[None]
    latent, lse_mqa = oracle.mla_decode(_problem(q_abs, [rows], rng=rng, scale=scale), lib=lib)
    o_mqa = mha.up_project(latent[0], W_UV)
    assert np.allclose(lse_mqa[0], lse_mha, rtol=0, atol=1e-12), (lse_mqa, lse_mha)
    err = np.abs(o_mqa - o_mha).max() / np.abs(o_mha).max()
    assert err < 1e-12, err


def pin_shift_invariance(lib):
    """Adding c to every score shifts lse by c and leaves out unchanged; with
    c in the thousands this also needs exp() evaluated stably."""
    rng = np.random.default_rng(15)
    L = 50
    rows = _rand_rows(rng, L)
    rows[:, D - 1] = _bf16_bits(np.ones(1, np.float32))[0]  # last rope column = 1
    q = _rand_q(rng, 1, 2)
    q[..., D - 1] = 0.0
    scale = 0.125
    o0, l0 = oracle.mla_decode(_problem(q, [rows], scale=scale, rng=np.random.default_rng(1)), lib=lib)
    for c in (3000.0, -3000.0):
        qc = q.copy()
        qc[..., D - 1] = c / scale  # exact: a power-of-two scale
        oc, lc = oracle.mla_decode(_problem(qc, [rows], scale=scale, rng=np.random.default_rng(1)), lib=lib)
        assert np.all(np.isfinite(lc)) and np.all(np.isfinite(oc)), "overflow in exp"
        assert np.abs(lc - (l0 + c)).max() < 1e-9, (lc, l0 + c)
        assert np.abs(oc - o0).max() < 1e-12


# ---------------------------------------------------------------- split and merge

def pin_split_merge(lib):
    rng = np.random.default_rng(8)
    lens = [1, 17, 64, 200]
    rows = [_rand_rows(rng, L) for L in lens]
    q = _rand_q(rng, len(lens), 3)
    p = _problem(q, rows, page_size=16, scale=0.09, rng=rng)
    full_o, full_l = oracle.mla_decode(p, lib=lib, nthreads=2)
    for S in (1, 2, 3, 7, 64):
        rb, rn, t0, t1 = [], [], [], []
        for b, L in enumerate(lens):
            cuts = np.sort(rng.integers(0, L + 1, S - 1)) if S > 1 else np.zeros(0, int)
            bounds = np.concatenate([[0], cuts, [L]])
            for n in range(3):
                for s in range(S):
                    rb.append(b); rn.append(n); t0.append(bounds[s]); t1.append(bounds[s + 1])
        po, pl = oracle.attend_spans(p, rb, rn, t0, t1, lib=lib, nthreads=2)
        po = po.reshape(len(lens), 3, S, DV)
        pl = pl.reshape(len(lens), 3, S)
        mo, ml = oracle.merge_states(po, pl, lib=lib)
        assert np.abs(ml - full_l).max() < 1e-12, S
        assert np.abs(mo - full_o).max() < 1e-12, S


def pin_merge_neutral(lib):
    rng = np.random.default_rng(10)
    o = rng.standard_normal((5, 1, 8))
    l = rng.standard_normal((5, 1))
    po = np.concatenate([o, np.zeros((5, 1, 8))], axis=1)
    pl = np.concatenate([l, np.full((5, 1), -np.inf)], axis=1)
    mo, ml = oracle.merge_states(po, pl, lib=lib)
    assert (mo == o[:, 0]).all() and (ml == l[:, 0]).all(), "(0, -inf) must carry no weight"
    mo, ml = oracle.merge_states(np.zeros((2, 3, 8)), np.full((2, 3), -np.inf), lib=lib)
    assert (mo == 0).all() and np.isneginf(ml).all()


def pin_empty_request(lib):
    rng = np.random.default_rng(11)
    q = _rand_q(rng, 3, 2)
    rows = [_rand_rows(rng, 0), _rand_rows(rng, 5), _rand_rows(rng, 0)]
    out, lse = oracle.mla_decode(_problem(q, rows, rng=rng), lib=lib)
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert np.isneginf(lse[0]).all() and np.isneginf(lse[2]).all()
    assert np.isfinite(lse[1]).all()


# ---------------------------------------------------------------- paging, fp8

def pin_page_permutation(lib):
    rng = np.random.default_rng(12)
    lens = [50, 129]
    rows = [_rand_rows(rng, L) for L in lens]
    q = _rand_q(rng, 2, 3)
    a = oracle.mla_decode(_problem(q, rows, page_size=16, rng=np.random.default_rng(1)), lib=lib)
    b = oracle.mla_decode(_problem(q, rows, page_size=16, rng=np.random.default_rng(2)), lib=lib)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all(), "result depends on physical page ids"
    # the same rows in pages of another size must also agree (exactly)
    c = oracle.mla_decode(_problem(q, rows, page_size=64, rng=np.random.default_rng(3)), lib=lib)
    assert (a[0] == c[0]).all() and (a[1] == c[1]).all()


def pin_fp8_cache(lib):
    rng = np.random.default_rng(13)
    L = 45
    codes = rng.integers(0, 256, (L, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes in the valid rows
    scale = 0.25
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * scale
    q = _rand_q(rng, 1, 2) * 0.05
    cache8, table, lens = _paged([codes], 16, np.random.default_rng(4),
                                 poison_bits=0x7F, dtype=np.uint8)
    p8 = oracle.Problem(q, cache8, table, lens, 0.1, cache_scale=scale)
    p16 = _problem(q, [_bf16_bits(vals.numpy())], page_size=16, scale=0.1,
                   rng=np.random.default_rng(4))
    o8, l8 = oracle.mla_decode(p8, lib=lib)
    o16, l16 = oracle.mla_decode(p16, lib=lib)
    assert (o8 == o16).all() and (l8 == l16).all(), "fp8 rows are not decoded x scale"


def pin_refuses_bad_tables(lib):
    rng = np.random.default_rng(14)
    q = _rand_q(rng, 1, 1)
    p = _problem(q, [_rand_rows(rng, 20)], rng=rng)
    p.block_table[0, 1] = p.num_blocks + 3
    try:
        oracle.mla_decode(p, lib=lib)
    except ValueError:
        return
    raise AssertionError("an out-of-range block id was accepted")


# ---------------------------------------------------------------- hand-worked

def _num(x):
    """Golden-file number: a float, "-inf", or {"ln": v} meaning ln(v)."""
    if isinstance(x, dict):
        return math.log(x["ln"])
    if x == "-inf":
        return -math.inf
    return float(x)


def pin_golden(lib):
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)
    for case in cases["decode"]:
        dqk, dv = case["dqk"], case["dv"]
        rows = np.array(case["rows"], dtype=np.float32)
        q = np.array(case["q"], dtype=np.float64)[None]
        p = _problem(q, [_bf16_bits(rows)], page_size=case["page_size"],
                     scale=case["scale"], rng=np.random.default_rng(0), dv=dv)
        out, lse = oracle.mla_decode(p, lib=lib, nthreads=1)
        want_out = np.array(case["out"], dtype=np.float64)
        assert np.allclose(out[0], want_out, rtol=0, atol=1e-12), (case["name"], out[0])
        want_lse = [_num(x) for x in case["lse"]]
        assert np.allclose(lse[0], want_lse, rtol=0, atol=1e-12), (case["name"], lse[0])
    for case in cases["merge"]:
        pl = np.array([[_num(x) for x in case["lse"]]])
        po = np.array([case["out"]], dtype=np.float64)
        mo, ml = oracle.merge_states(po, pl, lib=lib)
        assert np.allclose(mo[0], case["want_out"], rtol=0, atol=1e-12), case["name"]
        want = _num(case["want_lse"])
        assert (np.isneginf(ml[0]) and want == -math.inf) or abs(ml[0] - want) < 1e-12, case["name"]


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
