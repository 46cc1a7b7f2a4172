"""Seeded synthetic inputs for MLA decode, shared by the HIP path and the oracle.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the library tests and the oracle tests take their
inputs from here, so the oracle reads exactly the bytes the GPU reads.

Layouts follow the decode API of the pages (Model-Optimizer docs,
mla_attention_decode, "Parameters"): q [B, N, Lkv + R] with the absorbed
query cat[ql_nope, q_pe]; a paged latent cache [num_blocks, page_size,
Lkv + R] whose rows are cat[kv_c, k_pe]; block_table [B, max_blocks_per_seq];
seq_lens [B].

Recipe (the same for every workload):
  * values are float32 N(0, 1), rounded to bfloat16 (round-to-nearest-even);
  * the populated pages are assigned physical block ids by a random
    permutation; one extra block, the last, is a poison page filled with NaN;
  * block_table entries past a request's last page point at the poison page,
    and the unused rows of each request's last page are NaN too, so any read
    outside the valid rows shows up as NaN in the result;
  * for an fp8 cache the per-tensor scale is amax(|x|) / 448 over the populated
    rows, the cache stores x / scale rounded to OCP E4M3FN (saturated to
    +-448), NaN is 0x7F;
  * softmax_scale is float32(1 / sqrt(192)) = (P + R)^-1/2 for DeepSeek-V3's
    P = 128, R = 64, as the MLA layer computes it from its QK head width.
Random streams: numpy's PCG64 seeded with the workload seed for lengths and
permutations; values come from torch CPU generators seeded per 32768-row chunk
(seed * 1_000_003 + chunk), so generation is parallel and still deterministic.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

KV_LORA_RANK = 512      # Lkv, the latent width and the value/output width
QK_ROPE_HEAD_DIM = 64   # R, the decoupled RoPE width appended to the latent
HEAD_SIZE = KV_LORA_RANK + QK_ROPE_HEAD_DIM  # 576 = width of q and of a row

BF16_NAN_BITS = 0x7FC0
FP8_NAN_BITS = 0x7F
E4M3_MAX = 448.0

_CHUNK_ROWS = 32768


@dataclass
class Workload:
    name: str
    q: torch.Tensor             # bfloat16 [B, N, 576], CPU
    cache: torch.Tensor         # bfloat16 or uint8 [num_blocks, page, 576], CPU
    block_table: torch.Tensor   # int32 [B, max_blocks], CPU
    seq_lens: torch.Tensor      # int32 [B], CPU
    softmax_scale: float        # a float32 value
    cache_scale: float          # a float32 value; 1.0 for bf16
    cache_dtype: str            # "bf16" or "fp8_e4m3fn"
    num_kv_splits: int
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def N(self):
        return self.q.shape[1]

    @property
    def page_size(self):
        return self.cache.shape[1]

    def cache_bits(self) -> np.ndarray:
        """The raw cache bits: uint16 for bf16, uint8 for fp8."""
        if self.cache.dtype == torch.bfloat16:
            return self.cache.view(torch.int16).numpy().view(np.uint16)
        return self.cache.numpy()

    def q_float64(self) -> np.ndarray:
        """The bf16 query widened to float64 (exact)."""
        return self.q.to(torch.float64).numpy()

    def total_tokens(self) -> int:
        return int(self.seq_lens.to(torch.int64).sum())


# The five workloads: shapes, lengths and split counts of the pages'
# DeepSeek-V3-shaped decode (Lkv = 512, R = 64).
CONFIGS = {
    "tiny": dict(B=2, N=16, page_size=16, seq_lens=[37, 100], num_kv_splits=4,
                 cache_dtype="bf16", seed=1),
    "dsv3": dict(B=64, N=128, page_size=64, seq_lens=[4096] * 64, num_kv_splits=2,
                 cache_dtype="bf16", seed=2),
    "ragged": dict(B=128, N=128, page_size=64, seq_lens="uniform:1:32768",
                   num_kv_splits=32, cache_dtype="bf16", seed=3, max_len=32768),
    "long_context": dict(B=4, N=16, page_size=64, seq_lens=[131072] * 4,
                         num_kv_splits=64, cache_dtype="bf16", seed=4),
    "fp8_cache": dict(B=256, N=128, page_size=64, seq_lens=[8192] * 256,
                      num_kv_splits=1, cache_dtype="fp8_e4m3fn", seed=5),
}

DEFAULT_SOFTMAX_SCALE = float(np.float32(1.0 / math.sqrt(128 + 64)))


def draw_seq_lens(spec, B, seed):
    """Lengths: an explicit list, or "uniform:lo:hi" drawn from PCG64(seed)."""
    if isinstance(spec, str):
        kind, lo, hi = spec.split(":")
        assert kind == "uniform"
        rng = np.random.default_rng(seed)
        return rng.integers(int(lo), int(hi), size=B, endpoint=True).astype(np.int32)
    lens = np.asarray(spec, dtype=np.int32)
    assert lens.shape == (B,)
    return lens


def _normal_rows(seed: int, n_rows: int, width: int, threads: int):
    """float32 N(0,1) rows, generated in fixed chunks with per-chunk seeds."""
    chunks = [(c, min(_CHUNK_ROWS, n_rows - c * _CHUNK_ROWS))
              for c in range((n_rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS)]

    def one(ci):
        c, rows = ci
        g = torch.Generator().manual_seed(seed * 1_000_003 + c)
        return c, torch.randn(rows, width, generator=g, dtype=torch.float32)

    if threads <= 1 or len(chunks) <= 1:
        for ci in chunks:
            yield one(ci)
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        # bounded look-ahead keeps peak memory at a few chunks per thread
        pending = []
        it = iter(chunks)
        for ci in it:
            pending.append(ex.submit(one, ci))
            if len(pending) >= 2 * threads:
                yield pending.pop(0).result()
        for f in pending:
            yield f.result()


def make_workload(B, N, page_size, seq_lens, *, seed, num_kv_splits=1,
                  cache_dtype="bf16", max_len=None, name="custom",
                  softmax_scale=DEFAULT_SOFTMAX_SCALE, head_size=HEAD_SIZE,
                  threads=None, poison=True, perm_seed=None) -> Workload:
    """Build one seeded workload (see the module docstring for the recipe).

    max_len sets max_blocks_per_seq = ceil(max_len / page_size) (default: the
    longest drawn length, at least one page).  perm_seed (default seed + 7919)
    seeds the page permutation alone, so two workloads that differ only in it
    hold the same rows at different physical pages.
    """
    if cache_dtype not in ("bf16", "fp8_e4m3fn"):
        raise ValueError(cache_dtype)
    threads = threads or min(16, max(1, torch.get_num_threads()))
    lens = draw_seq_lens(seq_lens, B, seed)
    rng = np.random.default_rng(seed + 7919 if perm_seed is None else perm_seed)
    pages = (lens.astype(np.int64) + page_size - 1) // page_size
    total_pages = int(pages.sum())
    if max_len is None:
        max_len = int(lens.max()) if B else 0
    max_blocks = max(1, (int(max_len) + page_size - 1) // page_size)
    if B and pages.max() > max_blocks:
        raise ValueError("a length exceeds max_len")
    num_blocks = total_pages + 1
    poison_id = total_pages
    perm = rng.permutation(total_pages).astype(np.int32)

    block_table = np.full((B, max_blocks), poison_id, dtype=np.int32)
    page_start = np.concatenate([[0], np.cumsum(pages)]).astype(np.int64)
    for b in range(B):
        block_table[b, : pages[b]] = perm[page_start[b]: page_start[b + 1]]

    # physical row of every populated token, in request-major token order
    n_tok = int(lens.astype(np.int64).sum())
    lens64 = lens.astype(np.int64)
    tok_req = np.repeat(np.arange(B, dtype=np.int64), lens64)
    req_start = np.cumsum(lens64) - lens64
    tok_pos = np.arange(n_tok, dtype=np.int64) - np.repeat(req_start, lens64)
    phys_row = (perm[page_start[tok_req] + tok_pos // page_size].astype(np.int64)
                * page_size + tok_pos % page_size)
    phys_row_t = torch.from_numpy(phys_row)

    gq = torch.Generator().manual_seed(seed)
    q = torch.randn(B, N, head_size, generator=gq, dtype=torch.float32).to(torch.bfloat16)

    rows_total = num_blocks * page_size
    if cache_dtype == "bf16":
        fill = BF16_NAN_BITS if poison else 0
        cache = torch.full((rows_total, head_size), fill, dtype=torch.int16).view(torch.bfloat16)
        for c, vals in _normal_rows(seed, n_tok, head_size, threads):
            lo = c * _CHUNK_ROWS
            cache[phys_row_t[lo: lo + vals.shape[0]]] = vals.to(torch.bfloat16)
        cache_scale = 1.0
    else:
        vals_all = torch.empty((n_tok, head_size), dtype=torch.float32)
        for c, vals in _normal_rows(seed, n_tok, head_size, threads):
            lo = c * _CHUNK_ROWS
            vals_all[lo: lo + vals.shape[0]] = vals
        amax = float(vals_all.abs().max()) if n_tok else 1.0
        cache_scale = float(np.float32(np.float32(amax) / np.float32(E4M3_MAX)))
        fill = FP8_NAN_BITS if poison else 0
        cache = torch.full((rows_total, head_size), fill, dtype=torch.uint8)
        inv = torch.tensor(cache_scale, dtype=torch.float32)
        for lo in range(0, n_tok, _CHUNK_ROWS):
            blk = vals_all[lo: lo + _CHUNK_ROWS]
            code = (blk / inv).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
            cache[phys_row_t[lo: lo + blk.shape[0]]] = code.view(torch.uint8)
        del vals_all
    cache = cache.view(num_blocks, page_size, head_size)

    return Workload(
        name=name, q=q, cache=cache,
        block_table=torch.from_numpy(block_table),
        seq_lens=torch.from_numpy(lens.copy()),
        softmax_scale=float(np.float32(softmax_scale)),
        cache_scale=cache_scale, cache_dtype=cache_dtype,
        num_kv_splits=int(num_kv_splits), seed=int(seed),
        meta=dict(poison_block=poison_id, num_blocks=num_blocks,
                  max_blocks=max_blocks, max_len=int(max_len)))


def config_workload(name: str, **overrides) -> Workload:
    """One of the five named workloads (overrides replace any of its fields)."""
    spec = dict(CONFIGS[name])
    spec.update(overrides)
    B = spec.pop("B")
    N = spec.pop("N")
    P = spec.pop("page_size")
    lens = spec.pop("seq_lens")
    return make_workload(B, N, P, lens, name=name, **spec)


@dataclass
class InsertInputs:
    """One decode step's new-token data and a paged cache to insert it into."""
    ql_nope: torch.Tensor       # bfloat16 [T, N, 512], CPU
    q_pe: torch.Tensor          # bfloat16 [T, N, 64], CPU
    kv_c: torch.Tensor          # bfloat16 [T, 512], CPU
    k_pe: torch.Tensor          # bfloat16 [T, 64], CPU
    slot_mapping: torch.Tensor  # int64 [T], CPU; -1 marks a padding token
    cache: torch.Tensor         # bfloat16 or uint8 [num_blocks, page, 576], CPU
    cache_scale_inv: float      # a float32 value; 1.0 for bf16
    cache_dtype: str


def make_insert_inputs(T, N, num_blocks, page_size, *, seed, cache_dtype="bf16",
                       pad_every=0) -> InsertInputs:
    """Seeded inputs of a decode step's query concat and cache insert.

    Values are float32 N(0, 1) rounded to bfloat16, as for the workloads.  The
    T slots are distinct rows of the cache drawn by a random permutation;
    every pad_every-th token (if pad_every > 0) gets slot -1.  The cache starts
    with random contents: N(0, 1) bf16 values, or random E4M3FN codes other
    than NaN.  For an fp8 cache the per-tensor scale follows the workloads'
    convention, amax(|kv_c, k_pe|) / 448, and cache_scale_inv is its float32
    reciprocal (the caller pre-inverts it).
    """
    if cache_dtype not in ("bf16", "fp8_e4m3fn"):
        raise ValueError(cache_dtype)
    rows = num_blocks * page_size
    if T > rows:
        raise ValueError("more tokens than cache rows")
    g = torch.Generator().manual_seed(seed)
    ql_nope = torch.randn(T, N, KV_LORA_RANK, generator=g).to(torch.bfloat16)
    q_pe = torch.randn(T, N, QK_ROPE_HEAD_DIM, generator=g).to(torch.bfloat16)
    kv_c = torch.randn(T, KV_LORA_RANK, generator=g).to(torch.bfloat16)
    k_pe = torch.randn(T, QK_ROPE_HEAD_DIM, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(seed + 104729)
    slots = rng.permutation(rows)[:T].astype(np.int64)
    if pad_every > 0:
        slots[::pad_every] = -1
    if cache_dtype == "bf16":
        cache = torch.randn(num_blocks, page_size, HEAD_SIZE, generator=g).to(torch.bfloat16)
        inv = 1.0
    else:
        codes = torch.randint(0, 255, (num_blocks, page_size, HEAD_SIZE), generator=g)
        cache = torch.where(codes >= 0x7F, codes + 1, codes).to(torch.uint8)   # no 0x7F
        cache[cache == 0xFF] = 0xFE                                              # no 0xFF
        amax = float(torch.cat([kv_c.float().abs().flatten(), k_pe.float().abs().flatten()]).max()) \
            if T else 1.0
        scale = np.float32(np.float32(amax) / np.float32(E4M3_MAX))
        inv = float(np.float32(1.0) / scale)
    return InsertInputs(ql_nope=ql_nope, q_pe=q_pe, kv_c=kv_c, k_pe=k_pe,
                        slot_mapping=torch.from_numpy(slots), cache=cache,
                        cache_scale_inv=inv, cache_dtype=cache_dtype)


@dataclass
class GatherInputs:
    """A chunk of the requests' cached context, as a chunked prefill gathers it."""
    block_table: torch.Tensor   # int32 [B, max_blocks]
    cu_seq_lens: torch.Tensor   # int32 [B + 1]: request b's rows start at cu_seq_lens[b]
    token_to_seq: torch.Tensor  # int32 [num_tokens]
    seq_starts: torch.Tensor    # int32 [B]: first context token of the chunk, per request


def make_gather_inputs(wl: Workload, *, seed, chunk_tokens, align=True) -> GatherInputs:
    """One chunk over the workload's requests: request b contributes
    min(chunk_tokens, L_b - start_b) rows from a random start_b inside its
    context (a multiple of the page size when align is set, as the pages'
    gather requires; any token otherwise)."""
    rng = np.random.default_rng(seed)
    lens = wl.seq_lens.numpy().astype(np.int64)
    starts = np.zeros(wl.B, dtype=np.int64)
    counts = np.zeros(wl.B, dtype=np.int64)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        s = int(rng.integers(0, L))
        if align:
            s -= s % wl.page_size
        starts[b] = s
        counts[b] = min(int(chunk_tokens), int(L) - s)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    tts = np.repeat(np.arange(wl.B, dtype=np.int32), counts)
    return GatherInputs(block_table=wl.block_table, cu_seq_lens=torch.from_numpy(cu),
                        token_to_seq=torch.from_numpy(tts),
                        seq_starts=torch.from_numpy(starts.astype(np.int32)))


@dataclass
class MergeInputs:
    """Two partial attention states per (token, head), prefill layout."""
    prefix_out: torch.Tensor    # bfloat16 [T, N, D]
    prefix_lse: torch.Tensor    # float32 [N, T]
    suffix_out: torch.Tensor    # bfloat16 [T, N, D]
    suffix_lse: torch.Tensor    # float32 [N, T]


def make_merge_inputs(T, N, D, *, seed, empty_frac=0.1) -> MergeInputs:
    """Outputs N(0, 1) rounded to bf16; lse N(0, 3^2) in float32; a fraction
    empty_frac of the states of each side have lse = -inf (no weight), and
    the first token has both sides empty."""
    g = torch.Generator().manual_seed(seed)
    po = torch.randn(T, N, D, generator=g).to(torch.bfloat16)
    so = torch.randn(T, N, D, generator=g).to(torch.bfloat16)
    pl = torch.randn(N, T, generator=g) * 3
    sl = torch.randn(N, T, generator=g) * 3
    pl[torch.rand(N, T, generator=g) < empty_frac] = -float("inf")
    sl[torch.rand(N, T, generator=g) < empty_frac] = -float("inf")
    if T:
        pl[:, 0] = -float("inf")
        sl[:, 0] = -float("inf")
    return MergeInputs(prefix_out=po, prefix_lse=pl, suffix_out=so, suffix_lse=sl)


@dataclass
class ProjectionInputs:
    """Inputs of the per-head matmuls around the attention, in the pages' layouts."""
    q_nope: torch.Tensor        # bfloat16 [B, N, 128]
    latent_out: torch.Tensor    # bfloat16 [B, N, 512]
    W_UK: torch.Tensor          # bfloat16 [512, N, 128]  (Lkv, N, P)
    W_UV: torch.Tensor          # bfloat16 [512, N, 128]  (Lkv, N, V)


def make_projection_inputs(B, N, *, seed, P=128, V=128) -> ProjectionInputs:
    """Activations N(0, 1) and weights N(0, 1/Lkv) (so that products stay of
    order one), all rounded to bf16."""
    g = torch.Generator().manual_seed(seed)
    q_nope = torch.randn(B, N, P, generator=g).to(torch.bfloat16)
    latent = torch.randn(B, N, KV_LORA_RANK, generator=g).to(torch.bfloat16)
    s = 1.0 / math.sqrt(KV_LORA_RANK)
    W_UK = (torch.randn(KV_LORA_RANK, N, P, generator=g) * s).to(torch.bfloat16)
    W_UV = (torch.randn(KV_LORA_RANK, N, V, generator=g) * s).to(torch.bfloat16)
    return ProjectionInputs(q_nope=q_nope, latent_out=latent, W_UK=W_UK, W_UV=W_UV)
