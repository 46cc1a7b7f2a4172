"""fp64 CPU oracle for absorbed-query MLA decode (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and never imports it; both sides receive their inputs from the seeded
generators in ``head_latent_attention_decode_amd.workloads``, which hold none
of the method's arithmetic.

The arithmetic lives in ``mla_oracle.c`` (plain C, fp64, one (b, n) row at a
time) and, for the compute-friendly formulation used as an independent
cross-check, in ``mha.py`` (NumPy fp64).  See the header of ``mla_oracle.c``
for the passages of the pages each function follows.

Parity status: every exported function is pinned by ``tests/test_oracle_*.py``
(closed forms, brute force on 1-3 token contexts, the MHA == absorbed-MQA
identity, split+merge invariance, page-permutation invariance and the full
E4M3 code table).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "mla_oracle.c"
_LIB_PATH = _HERE / "liboracle_mla.so"

_lib = None


def build(src: Path | str = _SRC, out: Path | str = _LIB_PATH, extra_flags=()) -> Path:
    """Compile the C oracle with gcc into a shared library."""
    out = Path(out)
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-pthread",
           *extra_flags, str(src), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: Path | str | None = None):
    """Load (building first if absent) the oracle library; returns a ctypes CDLL."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
            build()
        path = _LIB_PATH
    lib = ctypes.CDLL(str(path))
    _declare(lib)
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _declare(lib):
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3fn_to_double.restype = ctypes.c_double
    lib.oracle_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
    common = [i32, i32, i32, i32, i32, i32, i32, i32,  # B N Dqk Dv P MB nb fp8
              P, P, ctypes.c_float, P, P, ctypes.c_float]
    lib.oracle_mla_decode.restype = i32
    lib.oracle_mla_decode.argtypes = common + [i32, P, P, P, P, i32]
    lib.oracle_mla_attend_spans.restype = i32
    lib.oracle_mla_attend_spans.argtypes = common + [i32, P, P, P, P, P, P, i32]
    lib.oracle_merge_states.restype = None
    lib.oracle_merge_states.argtypes = [i32, i32, i32, P, P, P, P]
    lib.oracle_e4m3fn_from_float.restype = ctypes.c_uint8
    lib.oracle_e4m3fn_from_float.argtypes = [ctypes.c_float]
    lib.oracle_gather.restype = i32
    lib.oracle_gather.argtypes = [i32, i32, P, i32, i32, i32, ctypes.c_float, P, i32, i32, P, P,
                                  P, P]
    lib.oracle_merge_two.restype = None
    lib.oracle_merge_two.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_concat_insert.restype = None
    lib.oracle_concat_insert.argtypes = [i32, i32, i32, i32, P, P, P, P, P, i32, i32, i32,
                                         ctypes.c_float, P, P]


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


class Problem:
    """The inputs exactly as the GPU reads them, as contiguous NumPy arrays.

    q:           float64 [B, N, Dqk]  (the bf16 query, converted exactly)
    cache:       uint16 [num_blocks, page_size, Dqk] (bf16 bits) or
                 uint8 (OCP E4M3FN bits)
    block_table: int32 [B, max_blocks]
    seq_lens:    int32 [B]
    """

    def __init__(self, q, cache, block_table, seq_lens, softmax_scale,
                 cache_scale=1.0, dv=512):
        self.q = np.ascontiguousarray(q, dtype=np.float64)
        self.cache = np.ascontiguousarray(cache)
        if self.cache.dtype not in (np.uint16, np.uint8):
            raise TypeError("cache must hold raw bf16 (uint16) or fp8 (uint8) bits")
        self.block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        self.seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        self.softmax_scale = float(np.float32(softmax_scale))
        self.cache_scale = float(np.float32(cache_scale))
        self.B, self.N, self.Dqk = self.q.shape
        self.num_blocks, self.page_size, dqk = self.cache.shape
        if dqk != self.Dqk:
            raise ValueError("query and cache widths differ")
        self.max_blocks = self.block_table.shape[1]
        self.Dv = int(dv)
        self.fp8 = 1 if self.cache.dtype == np.uint8 else 0

    def _common(self):
        return (self.B, self.N, self.Dqk, self.Dv, self.page_size,
                self.max_blocks, self.num_blocks, self.fp8,
                _ptr(self.q), _ptr(self.cache), self.cache_scale,
                _ptr(self.block_table), _ptr(self.seq_lens), self.softmax_scale)


def mla_decode(problem: Problem, rows=None, nthreads: int | None = None, lib=None):
    """Exact decode attention.  Returns (out float64, lse float64).

    rows=None: out [B, N, Dv], lse [B, N].  rows=(b_idx, n_idx): out [R, Dv],
    lse [R] for those (b, n) pairs only.
    """
    lib = lib or load()
    nthreads = nthreads or default_threads()
    p = problem
    if rows is None:
        out = np.empty((p.B, p.N, p.Dv), dtype=np.float64)
        lse = np.empty((p.B, p.N), dtype=np.float64)
        rc = lib.oracle_mla_decode(*p._common(), -1, None, None,
                                   _ptr(out), _ptr(lse), nthreads)
    else:
        rb = np.ascontiguousarray(rows[0], dtype=np.int32)
        rn = np.ascontiguousarray(rows[1], dtype=np.int32)
        out = np.empty((len(rb), p.Dv), dtype=np.float64)
        lse = np.empty((len(rb),), dtype=np.float64)
        rc = lib.oracle_mla_decode(*p._common(), len(rb), _ptr(rb), _ptr(rn),
                                   _ptr(out), _ptr(lse), nthreads)
    if rc != 0:
        raise ValueError(f"oracle refused the inputs (code {rc})")
    return out, lse


def attend_spans(problem: Problem, row_b, row_n, t0, t1, nthreads=None, lib=None):
    """Partial state (normalised out, natural-log lse) of rows over token spans."""
    lib = lib or load()
    nthreads = nthreads or default_threads()
    rb = np.ascontiguousarray(row_b, dtype=np.int32)
    rn = np.ascontiguousarray(row_n, dtype=np.int32)
    a = np.ascontiguousarray(t0, dtype=np.int64)
    z = np.ascontiguousarray(t1, dtype=np.int64)
    out = np.empty((len(rb), problem.Dv), dtype=np.float64)
    lse = np.empty((len(rb),), dtype=np.float64)
    rc = lib.oracle_mla_attend_spans(*problem._common(), len(rb), _ptr(rb), _ptr(rn),
                                     _ptr(a), _ptr(z), _ptr(out), _ptr(lse), nthreads)
    if rc != 0:
        raise ValueError(f"oracle refused the inputs (code {rc})")
    return out, lse


def merge_states(part_out, part_lse, lib=None):
    """S-way LSE merge.  part_out [..., S, Dv], part_lse [..., S] -> (out, lse)."""
    lib = lib or load()
    po = np.ascontiguousarray(part_out, dtype=np.float64)
    pl = np.ascontiguousarray(part_lse, dtype=np.float64)
    *lead, S, Dv = po.shape
    if tuple(pl.shape) != (*lead, S):
        raise ValueError("part_lse shape does not match part_out")
    R = int(np.prod(lead)) if lead else 1
    out = np.empty((*lead, Dv), dtype=np.float64)
    lse = np.empty(tuple(lead), dtype=np.float64)
    lib.oracle_merge_states(R, S, Dv, _ptr(po), _ptr(pl), _ptr(out), _ptr(lse))
    return out, lse


def bf16_to_double(bits: int, lib=None) -> float:
    return (lib or load()).oracle_bf16_to_double(bits)


def e4m3fn_to_double(bits: int, lib=None) -> float:
    return (lib or load()).oracle_e4m3fn_to_double(bits)


def e4m3fn_from_float(value: float, lib=None) -> int:
    """Nearest OCP E4M3FN code to the fp32 value (ties to even, saturating)."""
    return int((lib or load()).oracle_e4m3fn_from_float(float(np.float32(value))))


def concat_insert(ql_nope, q_pe, kv_c, k_pe, slot_mapping, cache, scale_inv=1.0, lib=None):
    """The decode step's query concat and cache insert (see mla_oracle.c).

    ql_nope uint16 [T, N, 512], q_pe uint16 [T, N, 64], kv_c uint16 [T, 512],
    k_pe uint16 [T, 64] (bf16 bits); slot_mapping int64 [T]; cache uint16
    (bf16 bits) or uint8 (E4M3FN codes) [num_blocks, page_size, 576], updated
    in place.  Returns q_out uint16 [T, N, 576].
    """
    ql_nope = np.ascontiguousarray(ql_nope, dtype=np.uint16)
    q_pe = np.ascontiguousarray(q_pe, dtype=np.uint16)
    kv_c = np.ascontiguousarray(kv_c, dtype=np.uint16)
    k_pe = np.ascontiguousarray(k_pe, dtype=np.uint16)
    slot = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    if not cache.flags["C_CONTIGUOUS"] or cache.dtype not in (np.uint16, np.uint8):
        raise TypeError("cache must be a contiguous uint16 or uint8 array")
    T, N, Dn = ql_nope.shape
    Dr = q_pe.shape[2]
    nb, P, D = cache.shape
    if D != Dn + Dr:
        raise ValueError("cache width must be Dn + Dr")
    q_out = np.zeros((T, N, D), dtype=np.uint16)
    (lib or load()).oracle_concat_insert(
        T, N, Dn, Dr, _ptr(ql_nope), _ptr(q_pe), _ptr(kv_c), _ptr(k_pe), _ptr(slot), nb, P,
        1 if cache.dtype == np.uint8 else 0, float(np.float32(scale_inv)), _ptr(cache),
        _ptr(q_out))
    return q_out


def gather(cache, block_table, cu_seq_lens, token_to_seq, seq_starts=None, scale=1.0, lib=None):
    """Chunked-context gather (see mla_oracle.c): returns uint16 bf16 bits
    [num_tokens, D].  cache: uint16 (bf16 bits) or uint8 (E4M3FN codes)
    [num_blocks, page_size, D].  Raises ValueError when a row's indices leave
    the table or the cache (such a row has no defined value)."""
    cache = np.ascontiguousarray(cache)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seq_lens, dtype=np.int32)
    tts = np.ascontiguousarray(token_to_seq, dtype=np.int32)
    st = None if seq_starts is None else np.ascontiguousarray(seq_starts, dtype=np.int32)
    nb, P, D = cache.shape
    n = tts.shape[0]
    if cu.shape != (bt.shape[0] + 1,) or (st is not None and st.shape != (bt.shape[0],)):
        raise ValueError("cu_seq_lens must be [B + 1] and seq_starts [B]")
    dst = np.zeros((n, D), dtype=np.uint16)
    rc = (lib or load()).oracle_gather(n, D, _ptr(cache), nb, P,
                                       1 if cache.dtype == np.uint8 else 0,
                                       float(np.float32(scale)), _ptr(bt), bt.shape[0],
                                       bt.shape[1], _ptr(cu), _ptr(tts),
                                       None if st is None else _ptr(st), _ptr(dst))
    if rc != 0:
        raise ValueError("oracle refused the gather: a row's owner, position, page or block "
                         "index leaves the table or the cache")
    return dst


def merge_two(prefix_out, prefix_lse, suffix_out, suffix_lse, lib=None):
    """Two-state merge: outputs [T, N, D], lse [N, T]; returns (out, lse) in fp64."""
    po = np.ascontiguousarray(prefix_out, dtype=np.float64)
    so = np.ascontiguousarray(suffix_out, dtype=np.float64)
    pl = np.ascontiguousarray(prefix_lse, dtype=np.float64)
    sl = np.ascontiguousarray(suffix_lse, dtype=np.float64)
    T, N, D = po.shape
    out = np.zeros((T, N, D))
    lse = np.zeros((N, T))
    (lib or load()).oracle_merge_two(T, N, D, _ptr(po), _ptr(pl), _ptr(so), _ptr(sl), _ptr(out),
                                     _ptr(lse))
    return out, lse


def mla_decode_multi(q, cache, block_table, seq_lens, softmax_scale, q_len, causal=True,
                     cache_scale=1.0, nthreads=None, lib=None):
    """Multi-token decode with a uniform query length (vLLM API docs,
    QueryLenSupport "UNIFORM"; causal or not among the new tokens).

    q float64 [B, q_len, N, Dqk]; seq_lens [B] count the q_len new tokens.
    Query row j of request b is an ordinary single-token decode row over the
    request's first L_b - (q_len - 1 - j) tokens when causal (its own token
    and those before it), over all L_b otherwise; a length below 0 is 0.
    Returns (out [B, q_len, N, Dv], lse [B, q_len, N]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, QL, N, D = q.shape
    if QL != q_len:
        raise ValueError("q's second axis must be q_len")
    lens = np.asarray(seq_lens, dtype=np.int64)
    row_lens = np.repeat(lens, q_len)
    if causal:
        row_lens = row_lens - (q_len - 1 - np.tile(np.arange(q_len), B))
    row_lens = np.maximum(row_lens, 0).astype(np.int32)
    prob = Problem(q.reshape(B * q_len, N, D), cache, np.repeat(np.asarray(block_table), q_len,
                                                                axis=0),
                   row_lens, softmax_scale, cache_scale)
    out, lse = mla_decode(prob, nthreads=nthreads, lib=lib)
    return out.reshape(B, q_len, N, -1), lse.reshape(B, q_len, N)
