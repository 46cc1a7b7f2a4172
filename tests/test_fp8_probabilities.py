"""Why the fp8-cache path keeps its probabilities in bf16 (a numerics study on
the CPU; no GPU and no library call).

PV on the fp8 MFMA would need P in E4M3 too.  The decode API of the
Model-Optimizer docs (mla_attention_decode, "Parameters": p_qdq) quantizes P
after the row sum, with the denominator left in full precision.  Here that
scheme is applied to rows of the fp8_cache workload (8192 tokens, E4M3 cache,
bf16 query), with the kernel's lazy running maximum (64-token tiles, a rescale
only when a tile's maximum exceeds the running one by 2^8, so P <= 256) and P
scaled by 448 / 256 into E4M3's range before rounding.  The PV sum uses the
rounded P, the row sum the fp32 P.  Against the exact fp64 attention, E4M3 P
leaves a row infinity-norm relative error near the fp8 tolerance (5e-2) on a
few hundred rows already, while bf16 P (what the kernel does) stays an order
of magnitude below it.
"""
import numpy as np
import torch

from head_latent_attention_decode_amd import workloads as W


def _e4m3(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).float().numpy()


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).bfloat16().float().numpy()


def _row_errors(requests=4, tile=64, headroom=8.0):
    wl = W.make_workload(requests, 128, 64, [8192] * requests, seed=5, cache_dtype="fp8_e4m3fn")
    K = (wl.cache.view(torch.float8_e4m3fn).float() * wl.cache_scale).numpy()
    bt = wl.block_table.numpy()
    q = wl.q.float().numpy()
    sl2 = np.float32(wl.softmax_scale * np.log2(np.e))
    sc = np.float32(448.0 / 256.0)
    errs = {"bf16": [], "e4m3": []}
    for b in range(requests):
        rows = K[bt[b, :128]].reshape(-1, 576)[:8192].astype(np.float64)
        x = (q[b].astype(np.float64) @ rows.T) * sl2
        w = np.exp2(x - x.max(1, keepdims=True))
        ref = (w @ rows[:, :512]) / w.sum(1, keepdims=True)
        m = np.full(128, -np.inf)
        num = {k: np.zeros((128, 512)) for k in errs}
        l = np.zeros(128)
        for t0 in range(0, 8192, tile):
            xt = x[:, t0:t0 + tile]
            mx = xt.max(1)
            if (mx > m + headroom).any():
                mn = np.maximum(m, mx)
                alpha = np.where(np.isinf(m), 0.0, np.exp2(m - mn))
                for k in num:
                    num[k] *= alpha[:, None]
                l *= alpha
                m = mn
            p = np.exp2(xt - m[:, None]).astype(np.float32)
            l += p.sum(1, dtype=np.float64)
            v = rows[t0:t0 + tile, :512]
            num["bf16"] += _bf16(p) @ v
            num["e4m3"] += (_e4m3(p * sc) / sc) @ v
        for k in num:
            out = num[k] / l[:, None]
            errs[k].extend(np.abs(out - ref).max(1) / np.abs(ref).max(1))
    return {k: np.array(v) for k, v in errs.items()}


def test_e4m3_probabilities_reach_the_fp8_tolerance():
    e = _row_errors()
    print(f"bf16 P max {e['bf16'].max():.4f}; E4M3 P max {e['e4m3'].max():.4f} over {e['bf16'].size} rows")
    assert e["bf16"].max() < 5e-3
    assert e["e4m3"].max() > 0.03           # within a factor 1.7 of 5e-2 on 512 rows
    assert e["e4m3"].max() > 8 * e["bf16"].max()
