#!/usr/bin/env python3
"""Benchmark of the exact-attention forward on one MI355X.

One step = one fa_fwd call over the whole batch of the workload (every step of
the hot path: work decomposition, K/V streaming, Q K^T, masked online softmax,
P V, epilogue with O and LSE), which is one attention-kernel launch. Inputs are
seeded synthetic data already resident in HBM when the timed region starts.
Prints ONE JSON line. The default workload is the largest configuration that
fits one GPU: causal attention at B=4, H=48, N=16384, d=64, fp16 (6.6 TFLOP per
launch); --workload picks another.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--splits S]
                  [--no-cpu-baseline] [--calibrate-copy] [--sweep]

--splits S cuts each Q-tile's keys into S chunks merged by their LSEs (fa_fwd_split; the
merge kernel is then part of the step); 0, the default, lets the library choose, which keeps
one chunk on grids that already fill the chip (the call is then fa_fwd); 1 never splits.
--sweep additionally prints one line per workload (for tables; not the bench line), and for
workloads the library splits, a second line without the split.
--bwd measures the backward pass (fa_bwd) on the workload instead and prints its own line:
one step = one fa_bwd call (row statistics, dK/dV and dQ kernels) with O and LSE from fa_fwd.
--calibrate-copy runs, after the timed region, one elementwise copy kernel of a known
size, used to scale the FETCH_SIZE / WRITE_SIZE hardware counters into bytes.
--variant V times another form of the forward on the workload's shape instead and prints its
own line (not the bench line): fp32 (the inputs kept in fp32: fa_fwd_ex on the fp32 matrix
cores, peak 157.3 TFLOP/s), fp8 (e4m3 inputs with per-tensor descales: fa_fwd_fp8, peak
5000), dropout (keep 0.9: fa_fwd_dropout) or alibi (an fp16 additive distance bias
-2^-3 |i - j| shared by the heads: fa_fwd_float_mask).

  python bench.py --summarize-counters FETCH_CSV WRITE_CSV --workload NAME --command CMD

reads the rocprofv3 counter collections of two such runs (one with FETCH_SIZE, one with
WRITE_SIZE) and records the attention kernel's HBM bytes per launch, scaled by what the
same counters read for the copy kernel (the last dispatch of each run), in
profiles/fa_fwd_hbm_counters.json, stamped with the hash of the kernel sources.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·d, causal halved) and % of MFMA peak, 1 GPU"
DEFAULT_WORKLOAD = "causal_b4_h48_n16384_d64_f16"
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # MI355X dense MFMA, fp16 / bf16
COUNTERS_FILE = os.path.join(ROOT, "profiles", "fa_fwd_hbm_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_114_amd", "csrc", f)
                  for f in ("fa_fwd_kernel.hpp", "fa_fwd_launch.hpp", "fa_fwd_inst.hip", "fa_fwd.hip", "fa_status.hpp")]


def kernel_source_hash(sources=None) -> str:
    """Hash of the forward kernel's sources with comments and blank lines removed, so that a
    change to the code (not to its comments) marks the recorded counters stale."""
    import re

    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None.

    None when no summary exists for this workload or when the kernel sources changed
    since the counters were taken (their hash is recorded with them).
    """
    try:
        with open(COUNTERS_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get("workloads", {}).get(workload)
    if not entry or data.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def to_device(bits, dtype_name, dev):
    import numpy as np
    import torch

    tdt = torch.float16 if dtype_name == "f16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)


def algorithmic_bytes(w) -> float:
    """Unique HBM bytes of one launch: Q, K, V read once, O (fp32) and LSE written once."""
    q = w.B * w.Hq * w.N * w.d * 2
    kv = 2 * w.B * w.Hkv * w.nk * w.d * 2
    o = w.B * w.Hq * w.N * w.d * 4
    lse = w.B * w.Hq * w.N * 4
    return float(q + kv + o + lse)


def planned_splits(w, splits: int) -> int:
    """The key-chunk count fa_fwd_split runs with for this request (1: no split)."""
    from exact_attention_114_amd import binding

    ws = binding.split_workspace_bytes(w.B, w.Hq, w.N, w.nk, w.d, splits)
    return ws // (w.B * w.Hq * w.N * (w.d + 1) * 4) if ws else 1


def time_gpu(w, steps: int, warmup: int, splits: int = 0, mask=None):
    """Seconds of wall time for `steps` forward calls, and the HIP-event average per call.
    mask: an optional uint8 [B or 1, Hq or 1, N, Nk] array passed to fa_fwd_mask."""
    import torch

    import exact_attention_114_amd as fa
    from exact_attention_114_amd import binding
    from exact_attention_114_amd import inputs as I

    dev = torch.device("cuda:0")
    qkv = I.workload_qkv(w)
    q, k, v = (to_device(x, w.dtype, dev) for x in (qkv.q, qkv.k, qkv.v))
    del qkv
    out = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    if mask is None:
        ws_bytes = binding.split_workspace_bytes(w.B, w.Hq, w.N, w.nk, w.d, splits)
    else:  # a [B or 1, Hq or 1, N, Nk] byte mask, contiguous
        ws_bytes = binding.mask_workspace_bytes(w.B, w.Hq, w.N, w.nk, w.d, splits,
                                                int(mask.shape[0] > 1), int(mask.shape[1] > 1))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    tm = None if mask is None else torch.from_numpy(mask).to(dev)

    # a square unmasked problem the plan does not split is one fa_fwd call
    plain = mask is None and w.window_left is None and w.nk == w.N and planned_splits(w, splits) == 1
    causal = w.causal if plain else False
    window = None if plain else w.band

    def call():
        fa.fwd(q, k, v, scale=w.scale, causal=causal, window=window, out=out, lse=lse,
               splits=None if plain else splits, workspace=ws, mask=tm, stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item(), "non-finite output"
    return wall, ev_ms / steps


VARIANT_PEAK = {"fp32": 157.3, "fp8": 5000.0, "dropout": 2500.0, "alibi": 2500.0}


def time_variant(w, variant: str, steps: int, warmup: int):
    """HIP-event milliseconds per forward call of the workload's shape in another form (the
    --variant option): fp32 inputs, fp8 inputs, dropout or an additive fp16 distance bias."""
    import torch

    import exact_attention_114_amd as fa
    from exact_attention_114_amd import inputs as I

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    window = w.band if (w.window_left is not None or w.nk != w.N) else None
    causal = w.causal if window is None else False
    if variant == "fp32":
        q, k, v = (torch.from_numpy(x).to(dev) for x in I.draw_qkv_f32(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed,
                                                                         w.k_mult, w.nk))

        def call():
            fa.fwd(q, k, v, scale=w.scale, causal=causal, window=window, stream=stream)
    elif variant == "fp8":
        (q8, k8, v8), ds = I.draw_qkv_fp8(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed, w.k_mult, w.nk)
        q, k, v = (torch.from_numpy(x).to(dev) for x in (q8, k8, v8))
        del q8, k8, v8

        def call():
            fa.fwd_fp8(q, k, v, *ds, scale=w.scale, causal=causal, window=window, stream=stream)
    elif variant in ("dropout", "alibi"):
        qkv = I.workload_qkv(w)
        q, k, v = (to_device(x, w.dtype, dev) for x in (qkv.q, qkv.k, qkv.v))
        del qkv
        mask = None
        if variant == "alibi":
            i = torch.arange(w.N, device=dev, dtype=torch.float32)[:, None] + (w.nk - w.N)
            j = torch.arange(w.nk, device=dev, dtype=torch.float32)[None, :]
            mask = (-0.125 * (i - j).abs()).to(torch.float16)[None, None].contiguous()
            if w.nk % 4:
                raise SystemExit("--variant alibi needs Nk a multiple of 4")

        def call():
            fa.fwd(q, k, v, scale=w.scale, causal=causal, window=window, stream=stream,
                   dropout=(0.9, 1234, 0) if variant == "dropout" else None, mask=mask)
    else:
        raise SystemExit(f"--variant {variant}: one of fp32, fp8, dropout, alibi")
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def bench_mask(w, kind: str):
    """A seeded byte mask for the workload and the FLOPs it leaves: 4 d per visible (query, key)
    pair, the band and the mask both applied.

    "document": each sequence packs documents of 1/8 to 1/2 of its length (drawn per batch
    element from PCG64(seed + 2000)); a query sees only keys of its own document, one
    [B, 1, N, N] mask shared by the heads.
    """
    import numpy as np

    from exact_attention_114_amd import inputs as I

    if kind != "document" or w.nk != w.N or w.window_left is not None:
        raise SystemExit(f"--mask {kind}: only 'document' on square unwindowed workloads")
    lens = I.document_lengths(w.B, w.N, w.seed + 2000, w.N // 8, w.N // 2)
    mask = I.document_mask(lens, w.N)
    pairs = 0
    for row in lens:
        for n in row:
            pairs += n * (n + 1) // 2 if w.causal else n * n
    return mask, 4.0 * w.Hq * w.d * pairs, lens


BWD_METRIC = "attention bwd TFLOP/s (10·B·H·N²·d, causal halved) and % of MFMA peak, 1 GPU"


def time_gpu_bwd(w, steps: int, warmup: int, mask=None):
    """Seconds of wall time for `steps` fa_bwd calls, and the HIP-event average per call.
    mask: an optional uint8 [B or 1, Hq or 1, N, Nk] array, passed to the forward that makes O
    and LSE and to fa_bwd_mask."""
    import torch

    import exact_attention_114_amd as fa
    from exact_attention_114_amd import binding
    from exact_attention_114_amd import inputs as I

    dev = torch.device("cuda:0")
    qkv = I.workload_qkv(w)
    q, k, v = (to_device(x, w.dtype, dev) for x in (qkv.q, qkv.k, qkv.v))
    del qkv
    dout = to_device(I.draw_dout(w.B, w.Hq, w.N, w.d, w.dtype, w.seed + 1000), w.dtype, dev)
    tm = None if mask is None else torch.from_numpy(mask).to(dev)
    o, lse = fa.fwd(q, k, v, scale=w.scale, window=w.band, mask=tm)
    if tm is None:
        ws_bytes = binding.bwd_workspace_bytes(w.B, w.Hq, w.N, w.d)
    else:
        ws_bytes = binding.bwd_mask_workspace_bytes(w.B, w.Hq, w.N, w.nk, w.d, int(mask.shape[0] > 1),
                                                    int(mask.shape[1] > 1))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    grads = (torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32, device=dev),
             torch.empty((w.B, w.Hkv, w.nk, w.d), dtype=torch.float32, device=dev),
             torch.empty((w.B, w.Hkv, w.nk, w.d), dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream(dev)

    def call():
        fa.bwd(q, k, v, o, lse, dout, scale=w.scale, window=w.band, workspace=ws, grads=grads, mask=tm,
               stream=stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert all(torch.isfinite(g).all().item() for g in grads), "non-finite gradient"
    return wall, ev0.elapsed_time(ev1) / steps


def bwd_algorithmic_bytes(w) -> float:
    """Unique HBM bytes of one fa_bwd call: Q, K, V, dO, LSE and O (fp32) read once; dQ, dK, dV
    (fp32) written once."""
    rd = w.B * w.Hq * w.N * w.d * (2 + 2 + 4) + 2 * w.B * w.Hkv * w.nk * w.d * 2 + w.B * w.Hq * w.N * 4
    wr = (w.B * w.Hq * w.N + 2 * w.B * w.Hkv * w.nk) * w.d * 4
    return float(rd + wr)


def bwd_line(w, args):
    mask, fwd_flops, doc_lens = (None, w.flops, None) if not args.mask else bench_mask(w, args.mask)
    wall, ms = time_gpu_bwd(w, args.steps, args.warmup, mask)
    flops = 2.5 * fwd_flops  # five products of the forward's size: S, dP, dV, dK, dQ
    value = flops * args.steps / wall / 1e12
    achieved = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    line = {
        "metric": BWD_METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs and dO; PCG64)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "Nk": w.nk, "d": w.d,
                   "causal": w.causal, "window_left": w.window_left, "in_dtype": w.dtype, "grad_dtype": "f32",
                   "o_dtype": "f32",
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "algorithmic_hbm_bytes": bwd_algorithmic_bytes(w), "call_ms": round(ms, 5),
                     "note": "achieved = algorithmic FLOP / HIP-event time of the whole fa_bwd call "
                             "(its kernels); per-kernel times are in the rocprofv3 summary"},
    }
    if mask is not None:
        line["config"]["mask"] = {"kind": args.mask, "shape": list(mask.shape),
                                  "documents_per_sequence": [len(r) for r in doc_lens],
                                  "visible_fraction": round(fwd_flops / w.flops, 5)}
    return line


COPY_BYTES = 64 * 1024 * 1024 * 4  # the calibration copy reads and writes this many bytes


def calibrate_copy():
    """One elementwise copy of a known size (256 MiB read + 256 MiB written) for counter scaling."""
    import torch

    n = COPY_BYTES // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    return n * 4


def cpu_baseline(w, budget_s: float = 12.0):
    """The fp64 oracle on a bounded sample of the workload, timed on the host cores.

    Units of 1024 query rows of one (batch, head) run on a process pool (one BLAS thread per
    process), batch element by batch element and head by head, in chunks of 2 units per core,
    until ``budget_s`` seconds have elapsed or the whole workload is done.
    """
    import numpy as np

    from exact_attention_114_amd import inputs as I
    from oracle.pool import attention_rows_pool, available_cores

    if w.window_left is not None or w.nk != w.N:
        return None  # the pooled oracle covers the causal and unmasked square forms; the bench line is GQA
    qkv = I.workload_qkv(w)
    # one process per core of the host, capped at 16: the CPU share of one GPU on the GPU machines
    host_cores = available_cores()
    cores = max(1, min(16, host_cores))
    rows_per_unit = 1024
    chunk = 2 * cores
    flops = 0.0
    n_units = 0
    elapsed = 0.0
    for b in range(w.B):
        q = I.bits_to_f64(qkv.q[b:b + 1], w.dtype)
        k = I.bits_to_f64(qkv.k[b:b + 1], w.dtype)
        v = I.bits_to_f64(qkv.v[b:b + 1], w.dtype)
        units = [(0, h, range(r0, min(w.N, r0 + rows_per_unit))) for h in range(w.Hq)
                 for r0 in range(0, w.N, rows_per_unit)]
        for c0 in range(0, len(units), chunk):
            part = units[c0:c0 + chunk]
            t0 = time.perf_counter()
            res = attention_rows_pool(q, k, v, I.scale_f32(w.scale), w.causal, part, cores)
            elapsed += time.perf_counter() - t0
            assert len(res) == len(part) and all(np.isfinite(r[3]).all() for r in res)
            for (_, _, rows) in part:
                r = np.arange(rows.start, rows.stop, dtype=np.float64)
                keys = (r + 1.0) if w.causal else np.full_like(r, float(w.N))
                flops += 4.0 * w.d * keys.sum()
            n_units += len(part)
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
    total_units = w.B * w.Hq * ((w.N + rows_per_unit - 1) // rows_per_unit)
    sample = (f"{n_units} of {total_units} units (1024 query rows of one head each, in batch/head order): "
              f"{flops / 1e9:.1f} GFLOP (causal-halved count) in {elapsed:.1f} s on a {cores}-process pool")
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "host_cores": host_cores,
            "kind": "oracle", "sample": sample + (f" (the pool is capped at 16 of the host's {host_cores} cores, "
                                                   "the CPU share of one GPU)" if host_cores > cores else "")}


def summarize_counters(fetch_csv: str, write_csv: str, workload: str, command: str) -> dict:
    """HBM bytes per launch of the attention kernel from two rocprofv3 --pmc collections.

    FETCH_SIZE and WRITE_SIZE are in KiB per dispatch. Each is scaled by the ratio of the
    copy kernel's known bytes to what the same counter reads for it (the copy is the last
    dispatch of the run), so a counter that misses part of the traffic is corrected.
    """
    import csv

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        fa = [float(r["Counter_Value"]) for r in rows if "fa_fwd_kernel" in r["Kernel_Name"]]
        copy_kib = float(rows[-1]["Counter_Value"])
        return fa, copy_kib

    fetch, fetch_copy = read(fetch_csv, "FETCH_SIZE")
    write, write_copy = read(write_csv, "WRITE_SIZE")
    fetch_scale = COPY_BYTES / (fetch_copy * 1024.0)
    write_scale = COPY_BYTES / (write_copy * 1024.0)
    fetch_kib = sum(fetch) / len(fetch)
    write_kib = sum(write) / len(write)
    entry = {"fetch_kib": round(fetch_kib, 3), "write_kib": round(write_kib, 3),
             "fetch_scale": round(fetch_scale, 5), "write_scale": round(write_scale, 5),
             "dispatches": [len(fetch), len(write)],
             "hbm_bytes_per_launch": round(fetch_kib * 1024.0 * fetch_scale + write_kib * 1024.0 * write_scale),
             "command": command}
    try:
        with open(COUNTERS_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    if data.get("kernel_source_hash") != kernel_source_hash():
        data = {"kernel_source_hash": kernel_source_hash(), "workloads": {}}
    data["workloads"][workload] = entry
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    with open(COUNTERS_FILE, "w") as f:
        json.dump(data, f, indent=1)
    return entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--bwd", action="store_true")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--mask", default="", help="'document': packed-document byte mask (fa_fwd_mask)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--command", default="")
    ap.add_argument("--variant", default="", help="fp32, fp8, dropout or alibi: time that form instead")
    args = ap.parse_args()

    if args.summarize_counters:
        print(json.dumps(summarize_counters(*args.summarize_counters, args.workload, args.command)))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each (batch, head) unit is independent, so the path would shard across GPUs without communication). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from exact_attention_114_amd import binding
    from exact_attention_114_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    binding.load_library()  # fails loudly if the HIP library is missing

    w = I.WORKLOADS[args.workload]
    if args.variant:
        ms = time_variant(w, args.variant, args.steps, args.warmup)
        tf = w.flops / (ms * 1e-3) / 1e12
        peak = VARIANT_PEAK[args.variant]
        print(json.dumps({"variant": args.variant, "workload": w.name, "steps": args.steps, "ms": round(ms, 5),
                          "tflops": round(tf, 2), "peak": peak, "frac": round(tf / peak, 4)}), flush=True)
        return
    if args.bwd:
        if args.sweep:
            for name in I.WORKLOADS:
                wk = I.WORKLOADS[name]
                _, ms = time_gpu_bwd(wk, max(3, min(50, int(5e12 / wk.flops))), 2)
                tf = 2.5 * wk.flops / (ms * 1e-3) / 1e12
                print(json.dumps({"sweep_bwd": name, "ms": round(ms, 5), "tflops": round(tf, 2),
                                  "pct_peak": round(100 * tf / PEAK_TFLOPS[wk.dtype], 2)}), flush=True)
        print(json.dumps(bwd_line(w, args)), flush=True)
        if args.calibrate_copy:
            calibrate_copy()
        return
    if args.sweep:
        for name in I.WORKLOADS:
            wk = I.WORKLOADS[name]
            steps = max(5, min(200, int(2e13 / wk.flops)))
            tries = [args.splits] + ([1] if planned_splits(wk, args.splits) > 1 else [])
            for s in tries:
                _, ms = time_gpu(wk, steps, 3, s)
                tf = wk.flops / (ms * 1e-3) / 1e12
                print(json.dumps({"sweep": name, "splits": planned_splits(wk, s), "ms": round(ms, 5),
                                  "tflops": round(tf, 2), "pct_peak": round(100 * tf / PEAK_TFLOPS[wk.dtype], 2)}),
                      flush=True)

    torch.cuda.synchronize()
    mask, flops, doc_lens = (None, w.flops, None) if not args.mask else bench_mask(w, args.mask)
    wall, ms_launch = time_gpu(w, args.steps, args.warmup, args.splits, mask)
    value = flops * args.steps / wall / 1e12
    achieved = flops / (ms_launch * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    if args.calibrate_copy:
        calibrate_copy()
    ns = planned_splits(w, args.splits)
    # with split keys the attention kernel runs ns times the grid (tiles chosen for that grid)
    bm, bn, grid = binding.tile(w.B * ns, w.Hq, w.Hkv, w.N, w.d, w.causal,
                                binding.FA_F16 if w.dtype == "f16" else binding.FA_BF16)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), K x2; PCG64 seed %d)" % w.seed if w.k_mult != 1.0
        else "synthetic (seeded N(0,1); PCG64 seed %d)" % w.seed,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "Nk": w.nk, "d": w.d,
                   "causal": w.causal, "window_left": w.window_left, "in_dtype": w.dtype, "out_dtype": "f32",
                   "scale": w.scale, "key_splits": ns,
                   "block_m": bm, "block_n": bn, "grid": grid, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name),
                     "algorithmic_hbm_bytes": algorithmic_bytes(w),
                     "kernel_ms": round(ms_launch, 5)},
    }
    if mask is not None:
        line["config"]["mask"] = {"kind": args.mask, "shape": list(mask.shape),
                                  "documents_per_sequence": [len(r) for r in doc_lens],
                                  "visible_fraction": round(flops / w.flops, 5)}
        line["roofline"]["traffic"] = None
        line["roofline"]["algorithmic_hbm_bytes"] = algorithmic_bytes(w) + float(mask.size)
    if ns > 1:
        line["roofline"]["note"] = ("split keys: kernel_ms and achieved cover the attention kernel and the "
                                    "merge kernel together (HIP events around the whole call)")
    if not args.no_cpu_baseline and mask is None:  # the pooled oracle takes no mask
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
