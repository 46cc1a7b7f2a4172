"""The C-ABI library on the host (CPU only): it loads, exports every symbol
the header declares, and rejects invalid arguments before launching
anything.  No call here reaches the GPU."""
import ctypes
import re
from pathlib import Path

import pytest

from head_latent_attention_decode_amd import mla

HEADER = Path(__file__).resolve().parents[1] / "include" / "mla_decode.h"
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return mla.load()


def shape(**kw):
    s = dict(batch=2, num_heads=128, kv_lora_rank=512, qk_rope_head_dim=64, num_blocks=10,
             page_size=64, max_blocks_per_seq=4, cache_dtype=0)
    s.update(kw)
    return mla.DecodeShape(**s)


def decode(lib, shp, S=4, ws_bytes=1 << 30, q=FAKE, cache=FAKE, scale=None, bt=FAKE, sl=FAKE,
           out=FAKE, ws=FAKE):
    return lib.mla_decode(ctypes.byref(shp) if shp is not None else None, q, cache, scale, bt, sl,
                          0.07, S, ws, ws_bytes, out, None, None)


def test_exports_everything_declared(lib):
    names = declared_functions()
    assert set(names) == set(mla.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings(lib):
    for st in range(7):
        assert lib.mla_status_string(st).decode().startswith("MLA_")
    assert b"unknown" in lib.mla_status_string(99)


def test_workspace_size(lib):
    shp = shape(batch=3, num_heads=16)
    assert lib.mla_decode_workspace_size(ctypes.byref(shp), 1) == 0
    assert lib.mla_decode_workspace_size(ctypes.byref(shp), 5) == 3 * 16 * 5 * 513 * 4
    assert lib.mla_decode_workspace_size(ctypes.byref(shp), 0) == 0
    assert lib.mla_decode_workspace_size(ctypes.byref(shp), 257) == 0
    assert lib.mla_decode_workspace_size(None, 4) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=8), 3), (dict(num_heads=0), 2), (dict(batch=-1), 2),
    (dict(kv_lora_rank=256), 3), (dict(qk_rope_head_dim=32), 3),
    (dict(page_size=48), 3), (dict(page_size=8), 3), (dict(num_blocks=0), 2),
    (dict(max_blocks_per_seq=0), 2), (dict(cache_dtype=7), 3),
])
def test_bad_shapes(lib, kw, status):
    assert decode(lib, shape(**kw)) == status


def test_bad_arguments(lib):
    assert decode(lib, None) == 1
    assert decode(lib, shape(), q=None) == 1
    assert decode(lib, shape(), cache=None) == 1
    assert decode(lib, shape(), bt=None) == 1
    assert decode(lib, shape(), sl=None) == 1
    assert decode(lib, shape(), out=None) == 1
    assert decode(lib, shape(), S=0) == 4
    assert decode(lib, shape(), S=257) == 4
    # bf16 cache with a scale pointer, fp8 cache without one
    assert decode(lib, shape(), scale=FAKE) == 3
    assert decode(lib, shape(cache_dtype=1), scale=None) == 1
    # workspace missing or short
    assert decode(lib, shape(), ws=None) == 5
    assert decode(lib, shape(), ws_bytes=2 * 128 * 4 * 513 * 4 - 1) == 5


def test_empty_batch_is_a_noop(lib):
    # B == 0: nothing to launch, and no pointer is needed
    assert decode(lib, shape(batch=0), q=None, cache=None, bt=None, sl=None, out=None,
                  ws=None, ws_bytes=0) == 0


def test_merge_arguments(lib):
    """mla_merge_states(B, N, S, dv, part_out, part_lse, out, lse, stream)."""
    f = lib.mla_merge_states
    assert f(-1, 4, 4, 512, FAKE, FAKE, FAKE, None, None) == 2
    assert f(8, -1, 4, 512, FAKE, FAKE, FAKE, None, None) == 2
    assert f(8, 4, 0, 512, FAKE, FAKE, FAKE, None, None) == 4
    assert f(8, 4, 257, 512, FAKE, FAKE, FAKE, None, None) == 4
    assert f(8, 4, 4, 256, FAKE, FAKE, FAKE, None, None) == 3
    assert f(65536, 65536, 4, 512, FAKE, FAKE, FAKE, None, None) == 3   # B * N beyond int32
    assert f(8, 4, 4, 512, None, FAKE, FAKE, None, None) == 1
    assert f(8, 4, 4, 512, FAKE, FAKE, None, None, None) == 1
    assert f(0, 4, 4, 512, None, None, None, None, None) == 0
    assert f(8, 0, 4, 512, None, None, None, None, None) == 0


def test_partials_arguments(lib):
    g = lib.mla_decode_partials
    shp = shape()
    assert g(ctypes.byref(shp), FAKE, FAKE, None, FAKE, FAKE, 0.1, 4, FAKE, 10, None) == 5
    assert g(ctypes.byref(shp), FAKE, FAKE, None, FAKE, FAKE, 0.1, 0, FAKE, 1 << 30, None) == 4


def insert(lib, T=4, N=8, ql=FAKE, qp=FAKE, kv=FAKE, kp=FAKE, slots=FAKE, nb=10, P=64, dt=0,
           inv=None, cache=FAKE, q_out=FAKE):
    return lib.mla_concat_q_insert_cache(T, N, ql, qp, kv, kp, slots, nb, P, dt, inv, cache,
                                         q_out, None)


def test_insert_arguments(lib):
    """Every invalid call returns before a launch (the pointers are fake)."""
    assert insert(lib, T=-1) == 2 and insert(lib, N=-1) == 2
    assert insert(lib, nb=-1) == 2 and insert(lib, P=0) == 2
    assert insert(lib, dt=7) == 3
    assert insert(lib, T=0) == 0                       # nothing to do
    assert insert(lib, kv=None) == 1 and insert(lib, kp=None) == 1
    assert insert(lib, slots=None) == 1 and insert(lib, cache=None) == 1
    assert insert(lib, dt=1) == 1                      # fp8 needs cache_scale_inv
    assert insert(lib, ql=None) == 1 and insert(lib, qp=None) == 1
    assert insert(lib, q_out=None) == 1


def test_projection_arguments(lib):
    for f in (lib.mla_absorb_query, lib.mla_up_project):
        assert f(-1, 8, FAKE, 1024, 128, FAKE, FAKE, None) == 2
        assert f(4, 8, FAKE, -8, 128, FAKE, FAKE, None) == 2
        assert f(0, 8, None, 0, 0, None, None, None) == 0          # nothing to do
        assert f(4, 8, None, 1024, 128, FAKE, FAKE, None) == 1
        assert f(4, 8, FAKE, 1024, 128, None, FAKE, None) == 1
        assert f(4, 8, FAKE, 1024, 128, FAKE, None, None) == 1
        assert f(4, 8, FAKE, 1023, 128, FAKE, FAKE, None) == 3     # stride not a multiple of 8
        assert f(4, 8, ctypes.c_void_p(0x1008), 1024, 128, FAKE, FAKE, None) == 3  # alignment


def test_check_inputs_arguments(lib):
    """Host-side argument checks of the device input check (fake pointers:
    nothing is launched on an error)."""
    f = lib.mla_check_inputs
    shp = shape()
    assert f(None, FAKE, FAKE, FAKE, None) == 1
    assert f(ctypes.byref(shp), FAKE, FAKE, None, None) == 1
    assert f(ctypes.byref(shp), None, FAKE, FAKE, None) == 1
    assert f(ctypes.byref(shape(page_size=0)), FAKE, FAKE, FAKE, None) == 2
    assert f(ctypes.byref(shape(num_heads=24)), FAKE, FAKE, FAKE, None) == 3


def test_binding_checks_caller_outputs():
    """A caller-supplied output is written in full by the library, so the
    binding refuses one of the wrong size, dtype or layout before any call."""
    import torch
    from head_latent_attention_decode_amd import mla
    dev = torch.device("cpu")
    good = torch.empty((2, 16, 512), dtype=torch.bfloat16)
    mla._check_output("out", good, torch.bfloat16, (2, 16, 512), dev)
    for bad in (torch.empty((2, 16, 511), dtype=torch.bfloat16),
                torch.empty((2, 16, 512), dtype=torch.float32),
                torch.empty((2, 512, 16), dtype=torch.bfloat16).transpose(1, 2)):
        with pytest.raises(ValueError):
            mla._check_output("out", bad, torch.bfloat16, (2, 16, 512), dev)
    with pytest.raises(ValueError):
        mla._check_output("lse", torch.empty(2, 15), torch.float32, (2, 16), dev)
