"""The device-side input check (mla_check_inputs) through the C ABI: valid
inputs report nothing; each broken precondition is counted, located and
classified; table entries past a request's pages are never judged."""
import pytest
import torch

from head_latent_attention_decode_amd import mla
from head_latent_attention_decode_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(wl, seq_lens=None, block_table=None):
    q = wl.q.to(DEV)
    cache = wl.cache.to(DEV)
    bt = (wl.block_table if block_table is None else block_table).to(DEV)
    sl = (wl.seq_lens if seq_lens is None else seq_lens).to(DEV)
    st = mla.check_inputs(q, cache, bt, sl, cache_dtype=wl.cache_dtype)
    torch.cuda.synchronize()
    return st.cpu().tolist()


def test_valid_inputs_pass():
    lens = [1, 17, 64, 65, 300, 0, 1000] * 5          # 35 requests: several per wave
    wl = W.make_workload(len(lens), 16, 16, lens, seed=31)
    assert _run(wl) == [0, -1, 0]


def test_each_violation_is_reported():
    lens = [100, 40, 64, 7, 200]
    wl = W.make_workload(len(lens), 16, 16, lens, seed=32)
    nb = wl.cache.shape[0]
    MB, P = wl.block_table.shape[1], 16
    sl = wl.seq_lens.clone()
    sl[3] = MB * P + 1                                # longer than the table row
    assert _run(wl, seq_lens=sl) == [1, 3, 1]
    sl = wl.seq_lens.clone()
    sl[1] = -5
    assert _run(wl, seq_lens=sl) == [1, 1, 1]
    bt = wl.block_table.clone()
    bt[4, 2] = nb                                     # one past the pool
    bt[2, 0] = -1
    assert _run(wl, block_table=bt) == [2, 2, 2]
    sl = wl.seq_lens.clone()
    sl[0] = MB * P + 100
    assert _run(wl, seq_lens=sl, block_table=bt) == [3, 0, 3]


def test_padding_entries_are_not_judged():
    lens = [16, 33]
    wl = W.make_workload(2, 16, 16, lens, seed=33, max_len=128)
    bt = wl.block_table.clone()
    bt[0, 1:] = 10 ** 6                               # past request 0's one page
    bt[1, 3:] = -7                                    # past request 1's three pages
    assert _run(wl, block_table=bt) == [0, -1, 0]
    bt[1, 2] = -7                                     # request 1's third page
    assert _run(wl, block_table=bt) == [1, 1, 2]
