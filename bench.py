#!/usr/bin/env python3
"""Benchmark of the MLA decode step on one MI355X.

A step is one mla_decode call over one batch of the ragged decode workload
(the largest of the five that fits one GPU): B = 128 requests, N = 128 heads,
KV lengths drawn uniformly from [1, 32768] (seed 3), page size 64, bf16
query and cache, num_kv_splits = 32.  Other workloads via --workload
(dsv3, long_context, fp8_cache, tiny).  The call runs the split-KV attention
kernel, then the LSE merge kernel (one kernel when num_kv_splits == 1).
Inputs are synthetic (seeded), generated on the host and resident in HBM
before the timed region; three copies of the query, cache and page table are
rotated so that no step finds its KV rows in the 256 MB Infinity Cache left
behind by the previous step.

Timing: K steps run back to back with nothing recorded between them, and
the wall clock over them gives the step time.  Then the split kernel runs K
more times alone, back to back in groups of 20 with HIP events recorded on the
launch stream around each group, which gives its average launch duration for
the roofline (an event between two launches idles the GPU for ~5 us, so no
event sits between two timed launches).

Printed: one JSON line with the whole-call algorithmic bandwidth as `value`
(GB/s: every KV row read once, plus q, out, lse, page-table entries and
lengths), per-step time, TFLOP/s, the split kernel's roofline fraction and
the fp64 CPU oracle timed on a sample of the same workload, and the graphics
and memory clocks that amd-smi reports during the timed passes (clocks are
not locked on this part).  --op stream measures plain streaming reads of the
dsv3 KV volume, the attainable-read reference for the decode kernels.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from head_latent_attention_decode_amd import mla  # noqa: E402
from head_latent_attention_decode_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
KERNEL_GROUP = 20               # launches per event pair when timing one kernel
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = ("decode attention GB/s and TFLOP/s (% of HBM/MFMA roofline); "
          "µs per B×N×Skv step")
SPLIT_SRC = os.path.join(ROOT, "head_latent_attention_decode_amd", "csrc", "mla_decode.hip")


class ClockSampler:
    """The GPU's clock state while the timed steps run: a thread that reads
    amd-smi's GPU metrics (current graphics clock of each XCD, memory clock,
    clock lock) every 20 ms.  Clocks on this part are not locked by default
    and follow power and temperature, so a step's time depends on them.  The
    sample is None when amd-smi is unavailable or the device is ambiguous."""

    def __init__(self, period_s=0.02):
        import threading
        self.period = period_s
        self.samples = []
        self.locked = None
        self.mem_mhz = None
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        self._last_stamp = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if len(handles) != 1:
                raise RuntimeError(f"{len(handles)} GPUs visible to amd-smi")
            self._smi, self._handle = amdsmi, handles[0]
        except Exception as e:  # no amd-smi, or not one GPU: report no clocks
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        # the metrics table is refreshed by the firmware more slowly than it
        # is read here: keep a table only when its timestamp has moved, and
        # drop the first one, which may predate the timed work
        stamp = m.get("system_clock_counter")
        if stamp == self._last_stamp:
            return
        first = self._last_stamp is None
        self._last_stamp = stamp
        if first:
            return
        clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, int) and 0 < c < 65535]
        if clks:
            self.samples.append(sum(clks) / len(clks))
        if isinstance(m.get("current_uclk"), int):
            self.mem_mhz = m["current_uclk"]
        if isinstance(m.get("gfxclk_lock_status"), int):
            self.locked = bool(m["gfxclk_lock_status"])

    def _run(self):
        while not self._stop.wait(self.period):
            try:
                self._read()
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"
                return

    def __enter__(self):
        if self._handle is not None:
            import threading
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass
        return False

    def summary(self):
        if self._handle is None:
            return {"error": self.error}
        # the firmware refreshes the table about once per 0.5-1 s, so a short
        # run may see none
        return {"gfx_mhz": [round(float(v), 0) for v in self.samples[:50]],
                "mem_mhz": self.mem_mhz, "gfx_locked": self.locked,
                "source": "amd-smi GPU metrics tables refreshed during the two timed passes "
                          "(graphics clock: mean over the XCDs)"}


def algorithmic_bytes(wl) -> int:
    """Bytes the method must move once: each KV row read once (all heads share
    it), q, out (bf16), lse (fp32), the used page-table entries and the
    lengths, plus the fp8 scale."""
    esz = 1 if wl.cache_dtype == "fp8_e4m3fn" else 2
    lens = wl.seq_lens.to(torch.int64)
    kv = int(lens.sum()) * W.HEAD_SIZE * esz
    pages = int(((lens + wl.page_size - 1) // wl.page_size).sum())
    per_req = wl.N * W.HEAD_SIZE * 2 + wl.N * W.KV_LORA_RANK * 2 + wl.N * 4 + 4
    return kv + wl.B * per_req + 4 * pages + (4 if esz == 1 else 0)


def algorithmic_flops(wl) -> int:
    return 2 * (W.HEAD_SIZE + W.KV_LORA_RANK) * wl.N * wl.total_tokens()


def split_kernel_bytes(wl) -> int:
    """Algorithmic bytes of the split kernel alone: KV rows, q, page-table
    entries and lengths (its outputs are the partials, which are not
    algorithmic)."""
    esz = 1 if wl.cache_dtype == "fp8_e4m3fn" else 2
    lens = wl.seq_lens.to(torch.int64)
    pages = int(((lens + wl.page_size - 1) // wl.page_size).sum())
    return (int(lens.sum()) * W.HEAD_SIZE * esz + wl.B * (wl.N * W.HEAD_SIZE * 2 + 4)
            + 4 * pages)


def split_kernel_name(wl) -> str:
    """Symbol prefix of the split kernel (the dominant one) the library
    launches for this workload: N a multiple of 64: the role-split kernel
    (bf16 or fp8 cache); otherwise the 16-head kernel."""
    return "mla_split_ws" if wl.N % 64 == 0 else "mla_split_h16"


def source_hash() -> str:
    with open(SPLIT_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(wl):
    """HBM bytes per split-kernel launch (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    scaled by a copy-kernel calibration) from the committed counter summary
    for this kernel and workload, if it was taken on the current source."""
    path = os.path.join(ROOT, "profiles", f"{split_kernel_name(wl)}_{wl.name}_traffic.md")
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    fields = dict(re.findall(r"^(source_sha256_16|hbm_bytes_per_launch) = (\S+)$", text, re.M))
    if fields.get("source_sha256_16") != source_hash() or "hbm_bytes_per_launch" not in fields:
        return None
    return int(fields["hbm_bytes_per_launch"])


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, n_req: int):
    """The fp64 oracle on the first n_req requests (all heads), on every host
    core this process may use.  Returns the algorithmic GB/s of that sample."""
    import oracle  # test infrastructure; only this leg of the benchmark uses it
    cores = oracle.default_threads()
    n_req = min(n_req, wl.B)
    sub = W.Workload(name=wl.name, q=wl.q[:n_req], cache=wl.cache,
                     block_table=wl.block_table[:n_req], seq_lens=wl.seq_lens[:n_req],
                     softmax_scale=wl.softmax_scale, cache_scale=wl.cache_scale,
                     cache_dtype=wl.cache_dtype, num_kv_splits=wl.num_kv_splits, seed=wl.seed)
    prob = oracle.Problem(sub.q_float64(), sub.cache_bits(), sub.block_table.numpy(),
                          sub.seq_lens.numpy(), sub.softmax_scale, cache_scale=sub.cache_scale)
    t0 = time.perf_counter()
    oracle.mla_decode(prob, nthreads=cores)
    dt = time.perf_counter() - t0
    gbs = algorithmic_bytes(sub) / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n_req} of {wl.B} requests, all {wl.N} heads, "
                      f"{int(sub.seq_lens.sum())} KV tokens, {dt:.2f} s wall"}


class Step:
    """Pre-marshalled arguments of one mla_decode call (the timed step) and of
    its split-kernel launch on its own (mla_decode_partials, for the kernel's
    duration), so the Python side adds as little as possible per step."""

    def __init__(self, lib, d, wl, S, stream):
        self.lib = lib
        self.S = S
        # the launches below hold raw pointers: keep the tensors alive
        self.inputs = d
        B, N = wl.B, wl.N
        self.shape = mla.make_shape(d["q"], d["latent_cache"], d["block_table"], wl.cache_dtype)
        nws = B * N * S * (W.KV_LORA_RANK + 1)
        self.ws = torch.empty(nws, dtype=torch.float32, device=d["q"].device)
        self.out = torch.empty((B, N, W.KV_LORA_RANK), dtype=torch.bfloat16, device=d["q"].device)
        self.lse = torch.empty((B, N), dtype=torch.float32, device=d["q"].device)
        vp = ctypes.c_void_p
        part_lse = self.ws.data_ptr() + B * N * S * W.KV_LORA_RANK * 4
        scale_ptr = vp(d["cache_scale"].data_ptr()) if d["cache_scale"] is not None else None
        inputs = (ctypes.byref(self.shape), vp(d["q"].data_ptr()),
                  vp(d["latent_cache"].data_ptr()), scale_ptr,
                  vp(d["block_table"].data_ptr()), vp(d["seq_lens"].data_ptr()),
                  ctypes.c_float(wl.softmax_scale), S)
        self.decode_args = inputs + (vp(self.ws.data_ptr()), nws * 4, vp(self.out.data_ptr()),
                                     vp(self.lse.data_ptr()), vp(stream))
        self.split_args = inputs + (vp(self.ws.data_ptr()), nws * 4, vp(stream))
        self.merge_args = (B, N, S, W.KV_LORA_RANK, vp(self.ws.data_ptr()), vp(part_lse),
                           vp(self.out.data_ptr()), vp(self.lse.data_ptr()), vp(stream))

    def decode(self):
        """One step: the whole mla_decode call (split kernel, then the merge;
        one direct kernel when S == 1)."""
        st = self.lib.mla_decode(*self.decode_args)
        if st != 0:
            raise mla.MLAError(st, "mla_decode")

    def split(self):
        """The dominant kernel alone: the kernel mla_decode launches first (at
        S == 1 the only one)."""
        if self.S == 1:
            return self.decode()
        st = self.lib.mla_decode_partials(*self.split_args)
        if st != 0:
            raise mla.MLAError(st, "mla_decode_partials")

    def merge(self):
        if self.S == 1:
            return
        st = self.lib.mla_merge_states(*self.merge_args)
        if st != 0:
            raise mla.MLAError(st, "mla_merge_states")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="ragged", choices=sorted(W.CONFIGS))
    ap.add_argument("--splits", type=int, default=None, help="override num_kv_splits")
    ap.add_argument("--copies", type=int, default=3, help="input copies rotated across steps")
    ap.add_argument("--cpu-requests", type=int, default=16,
                    help="requests in the CPU-oracle sample (0 disables it)")
    ap.add_argument("--op", default="decode",
                    choices=["decode", "insert", "gather", "merge2", "multi", "absorb", "upproj",
                             "stream"],
                    help="decode: the attention step (default); insert: the decode step's "
                         "query concat and cache insert at the workload's B and N; gather: "
                         "the chunked-context gather of the workload's whole context; "
                         "merge2: the two-state merge of prefill partials; multi: "
                         "multi-token (speculative) decode with --qlen query rows per request; "
                         "absorb / upproj: the per-head W_UK_T / W_UV matmuls at the "
                         "workload's B and N; stream: plain 16-byte streaming reads of the "
                         "dsv3 KV volume (attainable HBM read bandwidth)")
    ap.add_argument("--qlen", type=int, default=4, help="query rows per request for --op multi")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy 1 GiB device-to-device 3 times (a known-size kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": src.numel() * 4, "launches": 3}))
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: --gpus {args.gpus} is not supported "
              "(the decode path is built and measured on one MI355X; see DESIGN.md for how "
              "it would shard)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.op == "insert":
        run_insert(args)
        return
    if args.op == "gather":
        run_gather(args)
        return
    if args.op == "merge2":
        run_merge2(args)
        return
    if args.op == "multi":
        run_multi(args)
        return
    if args.op in ("absorb", "upproj"):
        run_projection(args)
        return
    if args.op == "stream":
        run_stream(args)
        return

    wl = W.config_workload(args.workload)
    S = args.splits or wl.num_kv_splits
    lib = mla.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    copies = []
    for _ in range(max(1, args.copies)):
        d = dict(q=wl.q.to(dev), latent_cache=wl.cache.to(dev),
                 block_table=wl.block_table.to(dev), seq_lens=wl.seq_lens.to(dev),
                 cache_scale=(torch.tensor([wl.cache_scale], dtype=torch.float32, device=dev)
                              if wl.cache_dtype == "fp8_e4m3fn" else None))
        copies.append(Step(lib, d, wl, S, stream.cuda_stream))
    torch.cuda.synchronize()

    # untimed warmup, long enough for the GPU clocks to reach their steady
    # state under this load
    for i in range(args.warmup):
        copies[i % len(copies)].decode()
    torch.cuda.synchronize()

    # The timed region: K whole steps back to back, nothing between them (an
    # event recorded between two launches idles the GPU for ~5 us).
    K = args.steps
    first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    clocks = ClockSampler().__enter__()
    t0 = time.perf_counter()
    first.record(stream)
    for i in range(K):
        copies[i % len(copies)].decode()
    last.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K
    gpu_ms_per_step = first.elapsed_time(last) / K

    # The dominant kernel's launch duration: K more launches of it alone, back to
    # back in groups of KERNEL_GROUP with HIP events recorded on the launch
    # stream around each group (an event pair around every launch would add
    # its own idle time to each), rotating over the copies; the merges follow
    # each group outside the events.
    n_groups = max(1, K // KERNEL_GROUP)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_groups)]
    for g in range(n_groups):
        ev[g][0].record(stream)
        for i in range(KERNEL_GROUP):
            copies[i % len(copies)].split()
        ev[g][1].record(stream)
        for st in copies:
            st.merge()
    torch.cuda.synchronize()
    clocks.__exit__(None, None, None)
    split_each = np.array([a.elapsed_time(b) / KERNEL_GROUP for a, b in ev])
    split_ms = float(split_each.mean())
    nbytes = algorithmic_bytes(wl)
    flops = algorithmic_flops(wl)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    split_bytes = split_kernel_bytes(wl)
    call_gbs = split_bytes / (split_ms * 1e-3) / 1e9
    call_tflops = flops / (split_ms * 1e-3) / 1e12
    # The split kernel is bound by HBM when its arithmetic intensity is below
    # the bf16 ridge (312.5 flop/B), as for every bf16 workload here.
    ai = flops / split_bytes
    ridge = BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(call_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(call_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(call_tflops, 1),
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(call_tflops / BF16_MFMA_PEAK_TFLOPS, 4)}
    roof["traffic"] = measured_traffic(wl)
    roof["kernel"] = split_kernel_name(wl)
    roof["kernel_ms"] = round(split_ms, 5)
    roof["kernel_us_p10_p50_p90_of_groups"] = [round(float(v) * 1e3, 2)
                                               for v in np.percentile(split_each, [10, 50, 90])]

    cpu = cpu_baseline(wl, args.cpu_requests) if args.cpu_requests > 0 else None
    lens = wl.seq_lens
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "gpu_us_per_step": round(gpu_ms_per_step * 1e3, 2),
        "tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "decode_tokens_per_s": round(wl.B / (ms_per_step * 1e-3), 1),
        "kv_tokens_per_s": round(int(lens.sum()) / (ms_per_step * 1e-3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.cache_dtype == "bf16" else "fp8_e4m3fn cache, bf16 MFMA",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: B={wl.B} requests x N={wl.N} heads, "
                               f"KV lengths {int(lens.min())}..{int(lens.max())}, "
                               f"page {wl.page_size}, num_kv_splits={S}, "
                               f"{wl.cache_dtype} cache, q/row width 576, value width 512",
                   "batch": wl.B, "num_heads": wl.N, "kv_tokens": int(lens.sum()),
                   "num_kv_splits": S, "page_size": wl.page_size,
                   "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                   "input_copies_rotated": len(copies)},
        "clocks": clocks.summary(),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def run_insert(args):
    """The decode step's query concat + cache insert (mla_concat_q_insert_cache)
    for B new tokens of N heads into a cache of the workload's page shape.
    Algorithmic bytes: the two query halves read and the concatenated query
    written (T * N * 576 * 2 each), each new row read (576 * 2) and written
    (576 * esz), the slots (8 each) and, for fp8, the scale (4)."""
    spec = W.CONFIGS[args.workload]
    cache_dtype = spec.get("cache_dtype", "bf16")
    T, N, P = spec["B"], spec["N"], spec["page_size"]
    nb = max(T, 4096 // P) * 4
    dev = torch.device("cuda:0")
    copies = []
    for c in range(max(1, args.copies)):
        x = W.make_insert_inputs(T, N, nb, P, seed=4242 + c, cache_dtype=cache_dtype)
        d = dict(ql_nope=x.ql_nope.to(dev), q_pe=x.q_pe.to(dev), kv_c=x.kv_c.to(dev),
                 k_pe=x.k_pe.to(dev), latent_cache=x.cache.to(dev),
                 slot_mapping=x.slot_mapping.to(dev),
                 q_out=torch.empty(T, N, W.HEAD_SIZE, dtype=torch.bfloat16, device=dev))
        if cache_dtype == "fp8_e4m3fn":
            d["cache_scale_inv"] = torch.tensor([x.cache_scale_inv], dtype=torch.float32,
                                                device=dev)
            d["cache_dtype"] = cache_dtype
        copies.append((x, d))

    calls = [(lambda d=d: mla.concat_q_insert_cache(**d)) for _, d in copies]
    K = args.steps
    kernel_ms, wall = _time_graph(calls, args.warmup, K)
    esz = 1 if cache_dtype == "fp8_e4m3fn" else 2
    nbytes = T * N * W.HEAD_SIZE * 2 * 2 + T * W.HEAD_SIZE * (2 + esz) + T * 8 + \
        (4 if esz == 1 else 0)
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_requests > 0:
        import oracle
        x = copies[0][0]
        bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
        cache = (bits(x.cache) if esz == 2 else x.cache.numpy()).copy()
        oracle.load()
        c0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - c0 < 1.0 or reps == 0:
            oracle.concat_insert(bits(x.ql_nope), bits(x.q_pe), bits(x.kv_c), bits(x.k_pe),
                                 x.slot_mapping.numpy(), cache, x.cache_scale_inv)
            reps += 1
        cpu_s = (time.perf_counter() - c0) / reps
        cpu = {"value": round(nbytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "sample": f"the whole step ({T} tokens x {N} heads), "
                                           f"{reps} runs, {cpu_s * 1e3:.2f} ms each"}
    line = {
        "metric": "decode-step query concat + cache insert GB/s (% of HBM roofline)",
        "value": round(nbytes / (wall / K) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 5),
        "us_per_step": round(wall * 1e6 / K, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if esz == 2 else "bf16 in, fp8_e4m3fn cache",
        "data": "synthetic",
        "config": {"workload": f"insert: T={T} new tokens x N={N} heads, page {P}, "
                               f"{cache_dtype} cache ({args.workload} shapes)",
                   "tokens": T, "num_heads": N, "algorithmic_bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "mla_concat_insert", "kernel_ms": round(kernel_ms, 5)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _time_calls(calls, warmup, steps):
    """Warm up, time `steps` calls (rotating over `calls`) back to back on the
    wall clock, then `steps` more in groups of KERNEL_GROUP with HIP events on
    the current stream around each group.  Returns (mean event ms per call,
    wall s of the first pass); no event sits between two timed calls, because
    each one idles the GPU for a few microseconds."""
    stream = torch.cuda.current_stream(torch.device("cuda:0"))
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_groups = max(1, steps // KERNEL_GROUP)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_groups)]
    for g in range(n_groups):
        ev[g][0].record(stream)
        for i in range(KERNEL_GROUP):
            calls[i % len(calls)]()
        ev[g][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) / KERNEL_GROUP for a, b in ev])), wall


def _time_graph(calls, warmup, steps):
    """For kernels shorter than a host launch: warm up, capture `steps` calls
    (rotating over `calls`) in one HIP graph, replay it once untimed, then time
    one replay with HIP events on the replay stream.  Returns (ms per launch,
    wall s of the timed replay): back-to-back launches with no host gaps, so
    the average is the kernel's own duration plus the graph's launch spacing."""
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                calls[i % len(calls)]()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(torch.device("cuda:0"))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def _op_line(metric, nbytes, kernel_ms, wall, steps, warmup, kernel, workload, dtype, cpu,
             extra=None):
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    cfg = {"workload": workload, "algorithmic_bytes": nbytes}
    cfg.update(extra or {})
    return {
        "metric": metric, "value": round(nbytes / (wall / steps) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(wall * 1e3 / steps, 5), "us_per_step": round(wall * 1e6 / steps, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic", "config": cfg,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": kernel, "kernel_ms": round(kernel_ms, 5)},
        "cpu_baseline": cpu,
    }


def run_gather(args):
    """The chunked-context gather of the workload's whole context (one chunk
    covering every request from token 0): each row read once from the paged
    cache (576 * esz bytes) and written as bf16 (1152 bytes), plus the page
    table, offsets and row owners."""
    wl = W.config_workload(args.workload)
    dev = torch.device("cuda:0")
    lens = wl.seq_lens.to(torch.int64)
    cu = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(lens, 0)]).to(torch.int32)
    tts = torch.repeat_interleave(torch.arange(wl.B, dtype=torch.int32), lens)
    n = int(lens.sum())
    fp8 = wl.cache_dtype == "fp8_e4m3fn"
    cache = wl.cache.to(dev)
    d = dict(latent_cache=cache, block_table=wl.block_table.to(dev), cu_seq_lens=cu.to(dev),
             token_to_seq=tts.to(dev),
             dst=torch.empty(n, W.HEAD_SIZE, dtype=torch.bfloat16, device=dev))
    if fp8:
        d.update(cache_scale=torch.tensor([wl.cache_scale], dtype=torch.float32, device=dev),
                 cache_dtype=wl.cache_dtype)
    kernel_ms, wall = _time_calls([lambda: mla.gather_cache(**d)], args.warmup, args.steps)
    esz = 1 if fp8 else 2
    pages = int(((lens + wl.page_size - 1) // wl.page_size).sum())
    nbytes = n * W.HEAD_SIZE * (esz + 2) + 4 * pages + 4 * (wl.B + 1) + 4 * n
    cpu = None
    if args.cpu_requests > 0:
        import oracle
        k = min(args.cpu_requests, wl.B)
        bits = (lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16))
        cache_np = bits(wl.cache) if not fp8 else wl.cache.numpy()
        m = int(cu[k])
        c0 = time.perf_counter()
        oracle.gather(cache_np, wl.block_table.numpy()[:k], cu.numpy()[:k + 1],
                      tts.numpy()[:m], scale=wl.cache_scale)
        cpu_s = time.perf_counter() - c0
        sb = m * W.HEAD_SIZE * (esz + 2)
        cpu = {"value": round(sb / cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{k} of {wl.B} requests ({m} rows), {cpu_s:.2f} s"}
    line = _op_line("chunked-context gather GB/s (% of HBM roofline)", nbytes, kernel_ms, wall,
                    args.steps, args.warmup, "mla_gather",
                    f"gather: {wl.name} context, {wl.B} requests, {n} rows, page "
                    f"{wl.page_size}, {wl.cache_dtype} cache -> bf16 workspace",
                    "bf16" if not fp8 else "fp8_e4m3fn cache -> bf16", cpu, {"rows": n})
    print(json.dumps(line), flush=True)


def run_merge2(args):
    """The two-state merge of prefill partials: T = 8192 tokens x N = 128
    heads x D = 128 (DeepSeek-V3's v_head_dim) bf16 outputs and [N, T] fp32
    LSEs; both states read, the merged state written."""
    T, N, D = 8192, 128, 128
    dev = torch.device("cuda:0")
    copies = []
    for c in range(max(1, args.copies)):
        m = W.make_merge_inputs(T, N, D, seed=600 + c)
        dd = dict(prefix_out=m.prefix_out.to(dev), prefix_lse=m.prefix_lse.to(dev),
                  suffix_out=m.suffix_out.to(dev), suffix_lse=m.suffix_lse.to(dev))
        dd["out"] = torch.empty_like(dd["prefix_out"])
        dd["out_lse"] = torch.empty_like(dd["prefix_lse"])
        copies.append((m, dd))
    calls = [(lambda dd=dd: mla.merge_attn_states(**dd)) for _, dd in copies]
    kernel_ms, wall = _time_calls(calls, args.warmup, args.steps)
    nbytes = 3 * T * N * D * 2 + 3 * N * T * 4
    cpu = None
    if args.cpu_requests > 0:
        import oracle
        m = copies[0][0]
        k = 256
        c0 = time.perf_counter()
        oracle.merge_two(m.prefix_out[:k].double().numpy(), m.prefix_lse[:, :k].double().numpy(),
                         m.suffix_out[:k].double().numpy(), m.suffix_lse[:, :k].double().numpy())
        cpu_s = time.perf_counter() - c0
        sb = 3 * k * N * D * 2 + 3 * N * k * 4
        cpu = {"value": round(sb / cpu_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{k} of {T} tokens, all heads, {cpu_s:.2f} s"}
    line = _op_line("two-state LSE merge GB/s (% of HBM roofline)", nbytes, kernel_ms, wall,
                    args.steps, args.warmup, "mla_merge_two",
                    f"merge2: T={T} tokens x N={N} heads x D={D}, bf16 states, [N, T] lse",
                    "bf16 states, fp32 lse", cpu)
    print(json.dumps(line), flush=True)


def run_multi(args):
    """Multi-token (speculative) decode, causal, q_len query rows per request of
    the workload.  Algorithmic bytes: every KV row once (the rows of a request
    share it), the q_len * N queries and outputs, LSEs, page table, lengths;
    flops: 2 * (576 + 512) per head per visible token of each query row."""
    wl = W.config_workload(args.workload)
    QL = args.qlen
    S = args.splits or wl.num_kv_splits
    dev = torch.device("cuda:0")
    copies = []
    for c in range(max(1, args.copies)):
        g = torch.Generator().manual_seed(700 + c)
        q = torch.randn(wl.B, QL, wl.N, W.HEAD_SIZE, generator=g).to(torch.bfloat16).to(dev)
        d = dict(q=q, latent_cache=wl.cache.to(dev), block_table=wl.block_table.to(dev),
                 seq_lens=wl.seq_lens.to(dev), softmax_scale=wl.softmax_scale,
                 num_kv_splits=S, causal=True,
                 cache_scale=(torch.tensor([wl.cache_scale], dtype=torch.float32, device=dev)
                              if wl.cache_dtype == "fp8_e4m3fn" else None),
                 cache_dtype=wl.cache_dtype)
        d["out"] = torch.empty(wl.B, QL, wl.N, W.KV_LORA_RANK, dtype=torch.bfloat16, device=dev)
        d["lse"] = torch.empty(wl.B, QL, wl.N, dtype=torch.float32, device=dev)
        ws = mla.load().mla_decode_multi_workspace_size(
            ctypes.byref(mla.make_shape(q.view(wl.B, QL * wl.N, -1), d["latent_cache"],
                                        d["block_table"], wl.cache_dtype)), QL, S)
        d["workspace"] = torch.empty(max(1, int(ws)), dtype=torch.uint8, device=dev)
        copies.append(d)
    calls = [(lambda d=d: mla.mla_decode_multi(**d)) for d in copies]
    call_ms, wall = _time_calls(calls, args.warmup, args.steps)
    lens = wl.seq_lens.to(torch.int64)
    esz = 1 if wl.cache_dtype == "fp8_e4m3fn" else 2
    pages = int(((lens + wl.page_size - 1) // wl.page_size).sum())
    rows = wl.B * QL * wl.N
    nbytes = int(lens.sum()) * W.HEAD_SIZE * esz + rows * (W.HEAD_SIZE * 2 + W.KV_LORA_RANK * 2
                                                           + 4) + 4 * pages + 4 * wl.B
    vis = sum(max(0, int(L) - (QL - 1 - j)) for L in lens.tolist() for j in range(QL))
    flops = 2 * (W.HEAD_SIZE + W.KV_LORA_RANK) * wl.N * vis
    tflops = flops / (call_ms * 1e-3) / 1e12
    line = _op_line("multi-token decode TFLOP/s (% of bf16 MFMA roofline)", nbytes, call_ms,
                    wall, args.steps, args.warmup, "mla_decode_multi (split + merge)",
                    f"multi: {wl.name}, B={wl.B} requests x q_len={QL} causal x N={wl.N} "
                    f"heads, num_kv_splits={S}, {wl.cache_dtype} cache",
                    "bf16", None, {"q_len": QL, "algorithmic_flops": flops})
    line["roofline"] = {"bound": "mfma", "achieved": round(tflops, 1),
                        "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                        "kernel": "mla_decode_multi (split + merge)",
                        "kernel_ms": round(call_ms, 5),
                        "hbm_frac": round(nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    line["metric"] = "multi-token decode TFLOP/s (% of bf16 MFMA roofline)"
    line["value"] = round(flops / (wall / args.steps) / 1e12, 2)
    line["unit"] = "TFLOP/s"
    print(json.dumps(line), flush=True)


def run_projection(args):
    """The per-head matmul before (absorb: q_nope . W_UK_T, K = 128 -> 512) or
    after (upproj: latent . W_UV, K = 512 -> 128) the attention, for the
    workload's B tokens and N heads.  Algorithmic bytes: the weights once
    (N * K * M * 2), the activations in and the results out; flops 2 * B * N * K * M."""
    spec = W.CONFIGS[args.workload]
    B, N = spec["B"], spec["N"]
    dev = torch.device("cuda:0")
    absorb = args.op == "absorb"
    K, M = (128, W.KV_LORA_RANK) if absorb else (W.KV_LORA_RANK, 128)
    copies = []
    for c in range(max(1, args.copies)):
        x = W.make_projection_inputs(B, N, seed=800 + c)
        if absorb:
            d = (x.q_nope.to(dev), x.W_UK.permute(1, 2, 0).contiguous().to(dev))
        else:
            d = (x.latent_out.to(dev), x.W_UV.transpose(0, 1).contiguous().to(dev))
        out = torch.empty(B, N, M, dtype=torch.bfloat16, device=dev)
        copies.append((d, out))
    fn = mla.absorb_query if absorb else mla.up_project
    calls = [(lambda d=d, o=o: fn(d[0], d[1], out=o)) for d, o in copies]
    kernel_ms, wall = _time_graph(calls, args.warmup, args.steps)
    nbytes = N * K * M * 2 + B * N * (K + M) * 2
    flops = 2 * B * N * K * M
    name = "absorb (q_nope . W_UK_T)" if absorb else "up-projection (latent . W_UV)"
    line = _op_line(f"per-head {name} GB/s (% of HBM roofline)", nbytes, kernel_ms, wall,
                    args.steps, args.warmup, "mla_head_mm",
                    f"{args.op}: B={B} tokens x N={N} heads, K={K} -> M={M}, bf16, "
                    f"{args.workload} shapes", "bf16", None,
                    {"tokens": B, "num_heads": N, "algorithmic_flops": flops})
    line["roofline"]["tflops"] = round(flops / (kernel_ms * 1e-3) / 1e12, 2)
    print(json.dumps(line), flush=True)


def run_stream(args):
    """Attainable HBM read bandwidth: the streaming-read probe (16-byte
    nontemporal loads, 8 in flight per thread, grid-stride) over the dsv3 KV
    volume (64 requests x 4096 rows x 1152 bytes = 302 MB), three buffers
    rotated so that no launch finds its data in the 256 MB Infinity Cache,
    for a sweep of grid sizes.  The decode kernels read each KV row once, so
    this is the ceiling their KV stream can approach on this part.  It also
    reports one CU's request rate for L2-resident data (GB/s per CU), the
    ceiling of a burst of tile loads, beside the per-CU share of the best
    HBM stream."""
    from head_latent_attention_decode_amd import build as B
    if not B.PROBE_LIB.exists():
        raise RuntimeError(f"{B.PROBE_LIB} is missing: run __graft_entry__.build()")
    probe = ctypes.CDLL(str(B.PROBE_LIB))
    probe.hbm_stream_read.restype = ctypes.c_int
    probe.hbm_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    probe.hbm_stream_read_lds.restype = ctypes.c_int
    probe.hbm_stream_read_lds.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    nbytes = 64 * 4096 * W.HEAD_SIZE * 2
    bufs = [torch.full((nbytes // 4,), c + 1, dtype=torch.int32, device=dev) for c in range(3)]
    grids = [256, 512, 1024, 2048, 4096, 8192, 16384]
    sink = torch.zeros(max(grids), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    results = {}
    for grid in grids:
        calls = [(lambda b=b, g=grid: probe.hbm_stream_read(
            ctypes.c_void_p(b.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), g,
            ctypes.c_void_p(stream.cuda_stream))) for b in bufs]
        ms, wall = _time_calls(calls, args.warmup, args.steps)
        results[grid] = (ms, wall)
    # the decode kernels' load path: direct-to-LDS, 256 workgroups (one per
    # CU) with 1, 2 or 4 streaming waves
    lds_gbs = {}
    for active in (1, 2, 4):
        calls = [(lambda b=b, a=active: probe.hbm_stream_read_lds(
            ctypes.c_void_p(b.data_ptr()), nbytes, 256, a,
            ctypes.c_void_p(stream.cuda_stream))) for b in bufs]
        lms, _ = _time_calls(calls, args.warmup, args.steps)
        lds_gbs[f"{active}_waves_per_cu"] = round(nbytes / (lms * 1e-3) / 1e9, 1)
    # a CU's request rate when every request hits L2 (8 windows of 256 KB, one
    # per XCD slot), direct-to-LDS and into registers, 1 or 4 waves per CU:
    # the ceiling of a tile-load burst, next to the per-CU share of the HBM stream
    probe.l2_request_rate.restype = ctypes.c_int
    probe.l2_request_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    win = torch.full((8 * 256 * 1024 // 4,), 1, dtype=torch.int32, device=dev)
    n_batches = 600
    l2_rate = {}
    for lds, name in ((1, "direct_to_lds"), (0, "registers")):
        for active in (1, 4):
            calls = [lambda a=active, l=lds: probe.l2_request_rate(
                ctypes.c_void_p(win.data_ptr()), n_batches, 256, a, l,
                ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))]
            if calls[0]() != 0:
                raise RuntimeError("l2_request_rate rejected its arguments")
            rms, _ = _time_calls(calls, min(args.warmup, 50), min(args.steps, 200))
            moved = 256 * active * n_batches * 8 * 1024
            l2_rate[f"{name}_{active}_waves"] = round(moved / (rms * 1e-3) / 1e9 / 256, 2)
    best = min(results, key=lambda g: results[g][0])
    ms, wall = results[best]
    l2_rate["hbm_stream_share"] = round(nbytes / (ms * 1e-3) / 1e9 / 256, 2)
    line = _op_line("attainable HBM read GB/s (plain streaming read, % of HBM peak)", nbytes, ms,
                    wall, args.steps, args.warmup, "hbm_stream_read_kernel",
                    f"stream: 302 MB read once per launch (the dsv3 KV volume), 3 buffers "
                    f"rotated, 16-byte nontemporal loads, best of grids {grids} "
                    f"(256 threads each)", "u32x4 loads", None,
                    {"best_grid": best,
                     "gbs_by_grid": {g: round(nbytes / (results[g][0] * 1e-3) / 1e9, 1)
                                     for g in grids},
                     "direct_to_lds_gbs": lds_gbs,
                     "l2_request_rate_gbs_per_cu": l2_rate})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
