"""Python binding of the C ABI in include/mla_decode.h (argument marshalling only).

Every step of the computation runs in the HIP library; this module only turns
torch tensors into pointers and sizes, supplies the current HIP stream, and
raises when the library returns a non-OK status.  PyTorch provides device
memory and streams, nothing else.  There is no fallback: if the library is
missing, every call raises.

The operation is the decode of the data-movement-friendly MLA path (vLLM API
docs, vllm.model_executor.layers.attention.mla_attention, module docstring,
"Data-Movement Friendly Approach (i.e. forward_mqa)") with the functional
signature of mla_attention_decode (Model-Optimizer docs,
modelopt.torch.kernels.quantization.attention.mla): see include/mla_decode.h.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libmla_decode.so"
_lib = None

MLA_OK = 0
MLA_CACHE_BF16 = 0
MLA_CACHE_FP8_E4M3FN = 1
KV_LORA_RANK = 512
QK_ROPE_HEAD_DIM = 64
HEAD_SIZE = KV_LORA_RANK + QK_ROPE_HEAD_DIM
MAX_KV_SPLITS = 256

EXPORTED = ("mla_status_string", "mla_decode_workspace_size", "mla_decode",
            "mla_decode_partials", "mla_merge_states", "mla_concat_q_insert_cache",
            "mla_gather_cache", "mla_merge_attn_states", "mla_decode_multi_workspace_size",
            "mla_decode_multi", "mla_absorb_query", "mla_up_project", "mla_check_inputs",
            "mla_decode_noalloc")
MLA_ERR_SCRATCH_LIMIT = 7
NOALLOC_SCRATCH_BYTES = 160 << 20


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class DecodeShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("kv_lora_rank", ctypes.c_int32), ("qk_rope_head_dim", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("cache_dtype", ctypes.c_int32)]


def library_path() -> Path:
    return _LIB_PATH


def load(path: Path | str | None = None):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else _LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is missing: build it with head_latent_attention_decode_amd."
                           "build.build_library() (or __graft_entry__.build())")
    lib = ctypes.CDLL(str(p))
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_decode_workspace_size.restype = sz
    lib.mla_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeShape), i32]
    lib.mla_decode.restype = ctypes.c_int
    lib.mla_decode.argtypes = [ctypes.POINTER(DecodeShape), vp, vp, vp, vp, vp,
                               ctypes.c_float, i32, vp, sz, vp, vp, vp]
    lib.mla_decode_noalloc.restype = ctypes.c_int
    lib.mla_decode_noalloc.argtypes = [ctypes.POINTER(DecodeShape), vp, vp, vp, vp, vp,
                                       ctypes.c_float, i32, vp, vp, vp]
    lib.mla_decode_partials.restype = ctypes.c_int
    lib.mla_decode_partials.argtypes = [ctypes.POINTER(DecodeShape), vp, vp, vp, vp, vp,
                                        ctypes.c_float, i32, vp, sz, vp]
    lib.mla_merge_states.restype = ctypes.c_int
    lib.mla_merge_states.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.mla_decode_multi_workspace_size.restype = sz
    lib.mla_decode_multi_workspace_size.argtypes = [ctypes.POINTER(DecodeShape), i32, i32]
    lib.mla_decode_multi.restype = ctypes.c_int
    lib.mla_decode_multi.argtypes = [ctypes.POINTER(DecodeShape), i32, i32, vp, vp, vp, vp, vp,
                                     ctypes.c_float, i32, vp, sz, vp, vp, vp]
    for name in ("mla_absorb_query", "mla_up_project"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [i32, i32, vp, ctypes.c_int64, ctypes.c_int64, vp, vp, vp]
    lib.mla_gather_cache.restype = ctypes.c_int
    lib.mla_gather_cache.argtypes = [i32, vp, i32, i32, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.mla_merge_attn_states.restype = ctypes.c_int
    lib.mla_merge_attn_states.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.mla_concat_q_insert_cache.restype = ctypes.c_int
    lib.mla_concat_q_insert_cache.argtypes = [i32, i32, vp, vp, vp, vp, vp, i32, i32, i32, vp,
                                              vp, vp, vp]
    lib.mla_check_inputs.restype = ctypes.c_int
    lib.mla_check_inputs.argtypes = [ctypes.POINTER(DecodeShape), vp, vp, vp, vp]
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mla_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != MLA_OK:
        raise MLAError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _cache_dtype(latent_cache: torch.Tensor, cache_dtype):
    if cache_dtype is not None:
        if cache_dtype in ("bf16", MLA_CACHE_BF16, torch.bfloat16):
            return MLA_CACHE_BF16
        if cache_dtype in ("fp8_e4m3fn", MLA_CACHE_FP8_E4M3FN, torch.float8_e4m3fn):
            return MLA_CACHE_FP8_E4M3FN
        raise ValueError(f"unknown cache dtype {cache_dtype!r}")
    if latent_cache.dtype == torch.bfloat16:
        return MLA_CACHE_BF16
    if latent_cache.dtype == torch.float8_e4m3fn:
        return MLA_CACHE_FP8_E4M3FN
    # raw bytes are ambiguous (E4M3 or a packed 4-bit format): make the caller say
    raise ValueError("a uint8 cache needs an explicit cache_dtype")


def make_shape(q, latent_cache, block_table, cache_dtype=None) -> DecodeShape:
    if q.dim() != 3 or latent_cache.dim() != 3 or block_table.dim() != 2:
        raise ValueError("expected q [B, N, 576], latent_cache [blocks, page, 576], "
                         "block_table [B, max_blocks]")
    B, N, D = q.shape
    nb, P, Dc = latent_cache.shape
    if D != HEAD_SIZE or Dc != HEAD_SIZE:
        raise ValueError("query and cache rows must be 576 wide (512 latent + 64 rope)")
    if block_table.shape[0] != B:
        raise ValueError("block_table rows must equal the batch")
    return DecodeShape(B, N, KV_LORA_RANK, QK_ROPE_HEAD_DIM, nb, P, block_table.shape[1],
                       _cache_dtype(latent_cache, cache_dtype))


def workspace_size(shape: DecodeShape, num_kv_splits: int) -> int:
    return int(load().mla_decode_workspace_size(ctypes.byref(shape), int(num_kv_splits)))


def _check_inputs(q, latent_cache, block_table, seq_lens, cache_scale):
    for name, t in (("q", q), ("latent_cache", latent_cache), ("block_table", block_table),
                    ("seq_lens", seq_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if tuple(seq_lens.shape) != (int(q.shape[0]),):
        raise ValueError("seq_lens must hold one int32 length per request: shape [B]")
    if cache_scale is not None and (cache_scale.dtype != torch.float32 or
                                    cache_scale.device != q.device or cache_scale.numel() != 1):
        raise ValueError("cache_scale must be a one-element float32 tensor on q's device")


def _check_output(name, t, dtype, shape, device):
    """A caller-supplied output: the library writes it in full, so its size,
    dtype, layout and device must be exactly what the call produces."""
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or
            not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape "
                         f"{tuple(shape)} on {device}")


def mla_decode(q, latent_cache, block_table, seq_lens, softmax_scale, num_kv_splits, *,
               cache_scale=None, cache_dtype=None, out=None, lse=None, return_lse=True,
               workspace=None):
    """Decode attention: returns (out bf16 [B, N, 512], lse f32 [B, N] or None)."""
    _check_inputs(q, latent_cache, block_table, seq_lens, cache_scale)
    shape = make_shape(q, latent_cache, block_table, cache_dtype)
    B, N = shape.batch, shape.num_heads
    dev = q.device
    if out is None:
        out = torch.empty((B, N, KV_LORA_RANK), dtype=torch.bfloat16, device=dev)
    _check_output("out", out, torch.bfloat16, (B, N, KV_LORA_RANK), dev)
    if return_lse and lse is None:
        lse = torch.empty((B, N), dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    if lse is not None:
        _check_output("lse", lse, torch.float32, (B, N), dev)
    need = workspace_size(shape, num_kv_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().mla_decode(ctypes.byref(shape), _ptr(q), _ptr(latent_cache), _ptr(cache_scale),
                           _ptr(block_table), _ptr(seq_lens), float(softmax_scale),
                           int(num_kv_splits), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                           _stream(dev))
    _check(st, "mla_decode")
    return out, lse


def mla_decode_noalloc(q, latent_cache, block_table, seq_lens, softmax_scale, num_kv_splits, *,
                       out, lse=None, cache_scale=None, cache_dtype=None):
    """mla_decode through the allocation-free entry point: the library keeps
    the split partials in its static device scratch (MLA_NOALLOC_SCRATCH_BYTES),
    and the caller supplies out (bf16 [B, N, 512]) and, optionally, lse
    (f32 [B, N]); this wrapper allocates nothing either.  Calls that overlap
    on one device race on that scratch."""
    _check_inputs(q, latent_cache, block_table, seq_lens, cache_scale)
    shape = make_shape(q, latent_cache, block_table, cache_dtype)
    B, N = shape.batch, shape.num_heads
    _check_output("out", out, torch.bfloat16, (B, N, KV_LORA_RANK), q.device)
    if lse is not None:
        _check_output("lse", lse, torch.float32, (B, N), q.device)
    st = load().mla_decode_noalloc(ctypes.byref(shape), _ptr(q), _ptr(latent_cache),
                                   _ptr(cache_scale), _ptr(block_table), _ptr(seq_lens),
                                   float(softmax_scale), int(num_kv_splits), _ptr(out),
                                   _ptr(lse), _stream(q.device))
    _check(st, "mla_decode_noalloc")
    return out, lse


def check_inputs(q, latent_cache, block_table, seq_lens, *, cache_dtype=None, status=None):
    """Device-side check of the decode's data preconditions (mla_check_inputs):
    returns the int32 [3] device status (count of bad requests, the lowest
    one or -1, a bitmask: 1 = seq_len out of range, 2 = block id out of
    range).  Asynchronous: read it when needed."""
    shape = make_shape(q, latent_cache, block_table, cache_dtype)
    if status is None:
        status = torch.empty(3, dtype=torch.int32, device=q.device)
    if (block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or
            not block_table.is_contiguous() or not seq_lens.is_contiguous()):
        raise ValueError("block_table and seq_lens must be contiguous int32")
    _check(load().mla_check_inputs(ctypes.byref(shape), _ptr(block_table), _ptr(seq_lens),
                                   _ptr(status), _stream(q.device)), "mla_check_inputs")
    return status


def mla_decode_multi(q, latent_cache, block_table, seq_lens, softmax_scale, num_kv_splits, *,
                     causal=True, cache_scale=None, cache_dtype=None, out=None, lse=None,
                     return_lse=True, workspace=None):
    """Multi-token decode: q bf16 [B, q_len, N, 576] -> (out bf16 [B, q_len, N, 512],
    lse f32 [B, q_len, N] or None).  seq_lens count the q_len new tokens."""
    if q.dim() != 4:
        raise ValueError("q must be [B, q_len, N, 576]")
    B, QL, N, D = (int(x) for x in q.shape)
    _check_inputs(q, latent_cache, block_table, seq_lens, cache_scale)
    shape = make_shape(q.view(B, QL * N, D), latent_cache, block_table, cache_dtype)
    shape.num_heads = N
    dev = q.device
    if out is None:
        out = torch.empty((B, QL, N, KV_LORA_RANK), dtype=torch.bfloat16, device=dev)
    _check_output("out", out, torch.bfloat16, (B, QL, N, KV_LORA_RANK), dev)
    if return_lse and lse is None:
        lse = torch.empty((B, QL, N), dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    if lse is not None:
        _check_output("lse", lse, torch.float32, (B, QL, N), dev)
    need = int(load().mla_decode_multi_workspace_size(ctypes.byref(shape), QL,
                                                      int(num_kv_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().mla_decode_multi(ctypes.byref(shape), QL, 1 if causal else 0, _ptr(q),
                                 _ptr(latent_cache), _ptr(cache_scale), _ptr(block_table),
                                 _ptr(seq_lens), float(softmax_scale), int(num_kv_splits),
                                 _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse), _stream(dev))
    _check(st, "mla_decode_multi")
    return out, lse


def mla_decode_partials(q, latent_cache, block_table, seq_lens, softmax_scale, num_kv_splits, *,
                        cache_scale=None, cache_dtype=None, workspace=None):
    """The split stage alone: returns (part_out f32 [B, N, S, 512], part_lse f32 [B, N, S]).

    An empty chunk has part_lse = -inf and unwritten part_out rows."""
    _check_inputs(q, latent_cache, block_table, seq_lens, cache_scale)
    shape = make_shape(q, latent_cache, block_table, cache_dtype)
    B, N, S = shape.batch, shape.num_heads, int(num_kv_splits)
    count = B * N * S * (KV_LORA_RANK + 1)
    if workspace is None:
        workspace = torch.empty(count, dtype=torch.float32, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().mla_decode_partials(ctypes.byref(shape), _ptr(q), _ptr(latent_cache),
                                    _ptr(cache_scale), _ptr(block_table), _ptr(seq_lens),
                                    float(softmax_scale), S, _ptr(workspace), ws_bytes,
                                    _stream(q.device))
    _check(st, "mla_decode_partials")
    flat = workspace.view(torch.float32)[:count]
    part_out = flat[: B * N * S * KV_LORA_RANK].view(B, N, S, KV_LORA_RANK)
    part_lse = flat[B * N * S * KV_LORA_RANK:].view(B, N, S)
    return part_out, part_lse


def mla_merge_states(part_out, part_lse, *, out=None, lse=None, return_lse=True):
    """S-way LSE merge: part_out f32 [B, N, S, 512], part_lse f32 [B, N, S] ->
    (out bf16 [B, N, 512], lse f32 [B, N] or None).  A 3-D part_out [R, S, 512]
    is taken as B = R requests of one head each."""
    if part_out.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise ValueError("partials must be float32")
    if not (part_out.is_contiguous() and part_lse.is_contiguous()):
        raise ValueError("partials must be contiguous")
    if part_out.dim() not in (3, 4):
        raise ValueError("part_out must be [B, N, S, 512] (or [R, S, 512])")
    *lead, S, dv = (int(x) for x in part_out.shape)
    if tuple(part_lse.shape) != (*lead, S) or part_lse.device != part_out.device:
        raise ValueError("part_lse must be [..., S] matching part_out, on its device")
    B, N = (lead[0], lead[1]) if len(lead) == 2 else (lead[0], 1)
    dev = part_out.device
    if out is None:
        out = torch.empty((*lead, dv), dtype=torch.bfloat16, device=dev)
    _check_output("out", out, torch.bfloat16, (*lead, dv), dev)
    if return_lse and lse is None:
        lse = torch.empty(tuple(lead), dtype=torch.float32, device=dev)
    if not return_lse:
        lse = None
    if lse is not None:
        _check_output("lse", lse, torch.float32, tuple(lead), dev)
    st = load().mla_merge_states(B, N, S, dv, _ptr(part_out), _ptr(part_lse), _ptr(out),
                                 _ptr(lse), _stream(dev))
    _check(st, "mla_merge_states")
    return out, lse


def concat_q_insert_cache(ql_nope, q_pe, kv_c, k_pe, latent_cache, slot_mapping, *,
                          cache_scale_inv=None, cache_dtype=None, q_out=None):
    """Decode-step query concat and cache insert (mla_concat_q_insert_cache).

    ql_nope bf16 [T, N, 512], q_pe bf16 [T, N, 64], kv_c bf16 [T, 512],
    k_pe bf16 [T, 64], slot_mapping int64 [T]; latent_cache [num_blocks,
    page_size, 576] (bf16, or E4M3FN with cache_scale_inv, a 1-element f32
    tensor) is updated in place.  Returns q_out bf16 [T, N, 576].
    """
    T, N = int(ql_nope.shape[0]), int(ql_nope.shape[1])
    for name, t, shape in (("ql_nope", ql_nope, (T, N, KV_LORA_RANK)),
                           ("q_pe", q_pe, (T, N, QK_ROPE_HEAD_DIM)),
                           ("kv_c", kv_c, (T, KV_LORA_RANK)),
                           ("k_pe", k_pe, (T, QK_ROPE_HEAD_DIM))):
        if tuple(t.shape) != shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor of shape {shape}")
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    if latent_cache.dim() != 3 or latent_cache.shape[2] != HEAD_SIZE or \
            not latent_cache.is_contiguous():
        raise ValueError("latent_cache must be a contiguous [num_blocks, page_size, 576] tensor")
    dt = _cache_dtype(latent_cache, cache_dtype)
    if dt == MLA_CACHE_FP8_E4M3FN and (cache_scale_inv is None or
                                       cache_scale_inv.dtype != torch.float32):
        raise ValueError("an fp8 cache needs cache_scale_inv (float32, one element)")
    if q_out is None:
        q_out = torch.empty((T, N, HEAD_SIZE), dtype=torch.bfloat16, device=ql_nope.device)
    st = load().mla_concat_q_insert_cache(
        T, N, _ptr(ql_nope), _ptr(q_pe), _ptr(kv_c), _ptr(k_pe), _ptr(slot_mapping),
        int(latent_cache.shape[0]), int(latent_cache.shape[1]), dt,
        _ptr(cache_scale_inv) if dt == MLA_CACHE_FP8_E4M3FN else None, _ptr(latent_cache),
        _ptr(q_out), _stream(ql_nope.device))
    _check(st, "mla_concat_q_insert_cache")
    return q_out


def gather_cache(latent_cache, block_table, cu_seq_lens, token_to_seq, *, seq_starts=None,
                 cache_scale=None, cache_dtype=None, dst=None):
    """Chunked-context gather (mla_gather_cache): returns bf16 [num_tokens, 576]."""
    n = int(token_to_seq.shape[0])
    for name, t in (("block_table", block_table), ("cu_seq_lens", cu_seq_lens),
                    ("token_to_seq", token_to_seq)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    if seq_starts is not None and (seq_starts.dtype != torch.int32 or
                                   not seq_starts.is_contiguous()):
        raise ValueError("seq_starts must be a contiguous int32 tensor")
    B, MB = int(block_table.shape[0]), int(block_table.shape[1])
    if tuple(cu_seq_lens.shape) != (B + 1,):
        raise ValueError("cu_seq_lens must be [batch + 1]")
    dt = _cache_dtype(latent_cache, cache_dtype)
    if dt == MLA_CACHE_FP8_E4M3FN and cache_scale is None:
        raise ValueError("an fp8 cache needs cache_scale")
    if dst is None:
        dst = torch.empty((n, HEAD_SIZE), dtype=torch.bfloat16, device=latent_cache.device)
    st = load().mla_gather_cache(n, _ptr(latent_cache), int(latent_cache.shape[0]),
                                 int(latent_cache.shape[1]), dt,
                                 _ptr(cache_scale) if dt == MLA_CACHE_FP8_E4M3FN else None,
                                 _ptr(block_table), B, MB, _ptr(cu_seq_lens), _ptr(token_to_seq),
                                 _ptr(seq_starts), _ptr(dst), _stream(latent_cache.device))
    _check(st, "mla_gather_cache")
    return dst


def merge_attn_states(prefix_out, prefix_lse, suffix_out, suffix_lse, *, out=None, out_lse=None,
                      return_lse=True):
    """Two-state merge (mla_merge_attn_states): outputs bf16 [T, N, D], lse f32 [N, T].
    out / out_lse may be the prefix (or suffix) tensors themselves."""
    T, N, D = (int(x) for x in prefix_out.shape)
    for name, t, dt, shape in (("prefix_out", prefix_out, torch.bfloat16, (T, N, D)),
                               ("suffix_out", suffix_out, torch.bfloat16, (T, N, D)),
                               ("prefix_lse", prefix_lse, torch.float32, (N, T)),
                               ("suffix_lse", suffix_lse, torch.float32, (N, T))):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape}")
    if out is None:
        out = torch.empty_like(prefix_out)
    if return_lse and out_lse is None:
        out_lse = torch.empty_like(prefix_lse)
    st = load().mla_merge_attn_states(T, N, D, _ptr(prefix_out), _ptr(prefix_lse),
                                      _ptr(suffix_out), _ptr(suffix_lse), _ptr(out),
                                      _ptr(out_lse if return_lse else None),
                                      _stream(prefix_out.device))
    _check(st, "mla_merge_attn_states")
    return out, (out_lse if return_lse else None)


def _head_mm(name, x, w, K, M, out):
    if x.dim() != 3 or x.shape[2] != K or x.dtype != torch.bfloat16 or x.stride(2) != 1:
        raise ValueError(f"x must be bf16 [B, N, {K}] with unit stride on the last axis")
    B, N = int(x.shape[0]), int(x.shape[1])
    if tuple(w.shape) != (N, K, M) or w.dtype != torch.bfloat16 or not w.is_contiguous():
        raise ValueError(f"weight must be a contiguous bf16 [N, {K}, {M}] tensor")
    if out is None:
        out = torch.empty((B, N, M), dtype=torch.bfloat16, device=x.device)
    st = getattr(load(), name)(B, N, _ptr(x), int(x.stride(0)), int(x.stride(1)), _ptr(w),
                               _ptr(out), _stream(x.device))
    _check(st, name)
    return out


def absorb_query(q_nope, w_uk_t, out=None):
    """ql_nope [B, N, 512] = per head q_nope [B, N, 128] . w_uk_t [N, 128, 512]."""
    return _head_mm("mla_absorb_query", q_nope, w_uk_t, 128, KV_LORA_RANK, out)


def up_project(latent_out, w_uv, out=None):
    """out [B, N, 128] = per head latent_out [B, N, 512] . w_uv [N, 512, 128]."""
    return _head_mm("mla_up_project", latent_out, w_uv, KV_LORA_RANK, 128, out)
