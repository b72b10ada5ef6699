#!/usr/bin/env python3
"""Throughput of the SATA hot path on one MI355X.

One step = one causal prefill (state reset + sata_prefill) of the workload
prefill_d64_p4_bf16: batch 1, 8 heads, n = 65536 tokens, d_K = d_V = 64,
P = 4, bf16 q/k/v, fp32 state, chunk 128.  `value` is prefill tokens/s
(batch * n / step time) with inputs already resident in HBM.

Beside it the same JSON line carries
  - roofline: the dominant kernel (prefill scan) against the bf16 MFMA peak,
    its duration taken from HIP events the library records around each of
    its launches on the launch stream;
  - decode: workload decode_d64_p4_f32 (32 x 8 heads, state built by an
    fp32 prefill of 8192 tokens, then 1024 timed decode steps with fresh
    inputs), tokens/s = batch / step time, and its roofline against HBM;
    plus per-step latency after 8192-, 32768- and 65536-token prefixes;
  - extra: the other prefill workloads;
  - softmax_gap: the prefill's and the decode's outputs against exact softmax
    attention on the same inputs, on sampled rows;
  - roofline.mfma_loop_ceiling: the rate a plain loop of the scan's MFMA
    instruction reaches on this GPU, beside the published peak;
  - cpu_baseline: the fp64 oracle on the host's cores on a bounded sample of
    the prefill workload's rows (decode.cpu_baseline: of its decode rows).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Progress goes to stderr; stdout gets exactly one JSON line.
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

METRIC = "SATA tokens/sec (prefill, decode) at d_K=64 P=4; % of HBM / MFMA peak"
METRIC_WORKLOAD = "prefill_d64_p4_bf16"   # the prefill the metric is quoted on
BACKWARD_WORKLOADS = ("prefill_d64_p4_bf16", "prefill_d16_p4_f32", "prefill_d128_p4_bf16")
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 matrix / vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "constant_cost_attention_amd", "csrc")


def log(msg: str):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-flatness", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="only: time every (chunk, positions per update wavefront) of the bf16 prefill workloads")
    ap.add_argument("--backward-only", action="store_true",
                    help="only: the backward calls of the backward section (for kernel traces)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--traffic-run", action="store_true",
                    help="one launch of each timed kernel plus a 1 GiB copy, for rocprofv3 --pmc runs")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter CSVs of two --traffic-run passes into profiles/traffic.json")
    return ap.parse_args()


def source_sha(fname: str) -> str:
    with open(os.path.join(CSRC, fname), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel and
    workload, or None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel, {}).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_sha(rec["source"]):
        return None
    return rec.get("bytes_per_launch")


def features(d: int, P: int) -> int:
    return math.comb(d + P - 1, P - 1)


def prefill_flops(wl) -> float:
    """Algorithmic FLOPs of the chunk-state and readout contractions:
    4 m (d_V + 1) per head-token (state update and readout, normaliser column included)."""
    return 4.0 * features(wl.d_k, wl.P) * (wl.d_v + 1) * wl.batch * wl.heads * wl.n


DECODE_WINDOW = 64


def decode_read_bytes(wl, state_elem: int = 4) -> float:
    """Algorithmic HBM bytes of a deferred step's readout: every head's state
    read once, plus the query."""
    m = features(wl.d_k, wl.P)
    return float(wl.batch * wl.heads * (state_elem * m * (wl.d_v + 1) + 4 * wl.d_k))


def f16_low_features(wl) -> int:
    """Features an fp16 state keeps in fp32: orders 0 and 1, rounded up to 64."""
    return min(-(-(1 + wl.d_k) // 64) * 64, features(wl.d_k, wl.P))


def decode_bytes_f16_main(wl) -> float:
    """Algorithmic HBM bytes of one decode step's main kernel on an fp16 state:
    the binary16 words (features from m_low on) read and written once."""
    m = features(wl.d_k, wl.P) - f16_low_features(wl)
    return float(wl.batch * wl.heads * 2 * 2 * m * (wl.d_v + 1))


def decode_bytes(wl, state_elem: int = 4) -> float:
    """Algorithmic HBM bytes of one decode step: every head's state (fp32, or
    bf16 with state_elem = 2) read and written once, plus the token's fp32
    q, k, v in and out's write."""
    m = features(wl.d_k, wl.P)
    return float(wl.batch * wl.heads * (2 * state_elem * m * (wl.d_v + 1) + 4 * (2 * wl.d_k + 2 * wl.d_v)))


# ------------------------------------------------------------------ prefill

def upload(x):
    import numpy as np
    import torch
    def one(name):
        a = x.storage(name)
        if x.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()
    return one("q"), one("k"), one("v")


def time_prefill(sata, wl, q, k, v, steps: int, warmup: int):
    import torch
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    out = torch.empty(v.shape, dtype=v.dtype, device="cuda")
    for _ in range(warmup):
        sata.sata_state_reset(st)
        sata.sata_prefill(idx, st, q, k, v, out, chunk=wl.chunk)
    torch.cuda.synchronize()
    sata.sata_profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        sata.sata_state_reset(st)
        sata.sata_prefill(idx, st, q, k, v, out, chunk=wl.chunk)
    e1.record()
    torch.cuda.synchronize()
    sata.sata_profile_enable(False)
    ms = e0.elapsed_time(e1) / steps
    scan_ms, scan_n = sata.sata_profile_query("prefill_scan")
    comb_ms, comb_n = sata.sata_profile_query("prefill_combine")
    flops = prefill_flops(wl)
    launches_per_step = scan_n / steps
    scan_avg = scan_ms / scan_n
    achieved = (flops / launches_per_step) / (scan_avg * 1e-3) / 1e12
    res = {
        "workload": wl.name,
        "value": wl.batch * wl.n / (ms * 1e-3),
        "unit": "tokens/s",
        "ms_per_step": ms,
        "tflops_whole_call": flops / (ms * 1e-3) / 1e12,
        "roofline": {
            "bound": "mfma", "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS,
            "unit": "TFLOP/s", "kernel": "prefill_scan",
            "launches_per_step": launches_per_step, "avg_launch_ms": scan_avg,
            "flops_per_launch": flops / launches_per_step,
            "traffic": traffic_for("prefill_scan", wl.name),
        },
        "combine_ms_per_step": comb_ms / steps,
    }
    res["roofline"]["frac"] = res["roofline"]["achieved"] / res["roofline"]["peak"]
    st.free()
    idx.free()
    return res


# ------------------------------------------------------------------ decode

def build_state(sata, idx, wl, prefix: int, dtype: str, seed: int):
    """Fresh state filled by a causal prefill of `prefix` seeded device tokens."""
    import torch
    import synth_inputs as si
    st = sata.State(idx, wl.batch, wl.heads)
    step = 8192
    for t0 in range(0, prefix, step):
        n = min(step, prefix - t0)
        q, k, v = si.draw_qkv_device((wl.batch, wl.heads), n, wl.d_k, wl.d_v, seed + t0, dtype)
        out = torch.empty(v.shape, dtype=v.dtype, device="cuda")
        sata.sata_prefill(idx, st, q, k, v, out)
        del q, k, v, out
    torch.cuda.synchronize()
    return st


def time_decode(sata, idx, st, wl, steps: int, warmup: int, seed: int):
    import torch
    import synth_inputs as si
    q, k, v = si.draw_qkv_device((wl.batch, wl.heads), steps + warmup, wl.d_k, wl.d_v, seed, "f32")
    q, k, v = (t.permute(2, 0, 1, 3).contiguous() for t in (q, k, v))     # [steps, B, H, d]
    out = torch.empty((steps + warmup, wl.batch, wl.heads, wl.d_v), dtype=torch.float32, device="cuda")
    for t in range(warmup):
        sata.sata_decode_step(idx, st, q[t], k[t], v[t], out[t])
    torch.cuda.synchronize()
    sata.sata_profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(warmup, warmup + steps):
        sata.sata_decode_step(idx, st, q[t], k[t], v[t], out[t])
    e1.record()
    torch.cuda.synchronize()
    sata.sata_profile_enable(False)
    ms = e0.elapsed_time(e1) / steps
    kern = {}
    for name in ("decode_stream", "decode_finish", "decode_read", "decode_fold", "decode_low"):
        kms, kn = sata.sata_profile_query(name)
        if kn:
            kern[name] = (kms / kn, kn)
    return ms, kern


def backward_flops(wl) -> float:
    """Algorithmic FLOPs of the backward's prefill passes: two passes of P orders
    (the forward recompute and dv) and 2 (d_V + 1) pseudo-head passes of P - 1
    orders (dk, dq), each 4 m (d_V + 1) per head-token."""
    m_p = features(wl.d_k, wl.P)
    m_l = features(wl.d_k, wl.P - 1) if wl.P > 1 else 0
    per = 2 * 4 * m_p * (wl.d_v + 1) + 2 * (wl.d_v + 1) * 4 * m_l * (wl.d_v + 1)
    return float(per) * wl.batch * wl.heads * wl.n


def time_backward(sata, wl, steps: int):
    """Whole sata_prefill_backward calls (they synchronise) on seeded device inputs."""
    import torch
    import synth_inputs as si
    q, k, v = si.draw_qkv_device((wl.batch, wl.heads), wl.n, wl.d_k, wl.d_v, wl.seed, wl.dtype)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 77)
    dout = torch.randn(v.shape, generator=g, device="cuda", dtype=torch.float32).to(v.dtype)
    grads = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for _ in range(3)]
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    sata.sata_prefill_backward(idx, q, k, v, dout, *grads, chunk=wl.chunk)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        sata.sata_prefill_backward(idx, q, k, v, dout, *grads, chunk=wl.chunk)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    idx.free()
    del q, k, v, dout, grads
    torch.cuda.empty_cache()
    fl = backward_flops(wl)
    return {"workload": wl.name, "ms_per_call": ms, "value": wl.batch * wl.n / (ms * 1e-3),
            "unit": "tokens/s", "algorithmic_tflops": fl / (ms * 1e-3) / 1e12, "flops_per_call": fl,
            "timing": "host clock around whole calls (each call synchronises its stream)"}


def stream_ceiling(nbytes: float, reps: int = 10):
    """Reference rates of two plain torch kernels over a buffer the size of the
    decode workload's state (far larger than every cache): an in-place fp32
    scale (read and write once) and row sums over 4096-wide rows (read once),
    timed with events on torch's stream, in GB/s of algorithmic bytes.  They
    are points of comparison, not upper bounds: the library's read kernel
    streams faster than the torch read."""
    import torch
    x = torch.ones(int(nbytes) // 4 // 4096 * 4096, dtype=torch.float32, device="cuda")
    out = {}
    for name, fn, moved in (("torch_rmw_gbs", lambda: x.mul_(1.0), 2 * x.numel() * 4),
                            ("torch_read_gbs", lambda: x.view(-1, 4096).sum(1), x.numel() * 4)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = moved / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del x
    torch.cuda.empty_cache()
    out["method"] = ("reference rates (not upper bounds) of torch in-place mul_ and row sums of 4096 over a "
                     "%.2f GB fp32 tensor" % (nbytes / 1e9))
    return out


TILE_SWEEP = (("prefill_d64_p4_bf16", (64, 128), 2), ("prefill_d32_p4_bf16", (64, 128), 3),
              ("prefill_d16x64h_p4_bf16", (64, 128), 5), ("prefill_d128_p4_bf16", (64,), 1))


def tile_sweep(sata):
    """Whole-call ms of the fp16-operand scan's prefill for each chunk length and
    positions per update wavefront (the rule's choice and the other), per workload."""
    import dataclasses
    import torch
    import synth_inputs as si
    rows = []
    for name, chunks, mx in TILE_SWEEP:
        wl = si.WORKLOADS[name]
        q, k, v = si.draw_qkv_device((wl.batch, wl.heads), wl.n, wl.d_k, wl.d_v, wl.seed, wl.dtype)
        for c in chunks:
            for mt in sorted({1, mx}):
                sata.sata_debug_prefill_positions(mt)
                r = time_prefill(sata, dataclasses.replace(wl, chunk=c), q, k, v, 3, 1)
                rows.append({"workload": name, "chunk": c, "positions": mt, "ms_per_call": r["ms_per_step"],
                             "scan_ms": r["roofline"]["avg_launch_ms"]})
                log("tile sweep %s chunk %d positions %d: %.3f ms per call (scan %.3f)"
                    % (name, c, mt, r["ms_per_step"], r["roofline"]["avg_launch_ms"]))
        sata.sata_debug_prefill_positions(0)
        del q, k, v
        torch.cuda.empty_cache()
    return rows


def decode_section(sata, wl, steps: int, warmup: int, flatness: bool):
    import torch
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    log("decode: fp32 prefill of %d tokens x %d heads" % (wl.n, wl.batch * wl.heads))
    st = build_state(sata, idx, wl, wl.n, "f32", wl.seed)
    ms, kern = time_decode(sata, idx, st, wl, steps, warmup, wl.seed + 30)
    kern_ms, fin_ms = kern["decode_stream"][0], kern["decode_finish"][0]
    sth = sata.State(idx, wl.batch, wl.heads, dtype=torch.float16)
    sata.sata_state_convert(st, sth)
    log("decode: the same state converted to fp16 storage (orders 0 and 1 in fp32)")
    msh, kh = time_decode(sata, idx, sth, wl, steps, warmup, wl.seed + 30)
    kernh, finh, lowh = kh["decode_stream"][0], kh["decode_finish"][0], kh["decode_low"][0]
    sth.free()
    nbytesh = decode_bytes_f16_main(wl)
    achh = nbytesh / (kernh * 1e-3) / 1e9
    st16 = sata.State(idx, wl.batch, wl.heads, dtype=torch.bfloat16)
    sata.sata_state_convert(st, st16)
    st.free()
    log("decode: the same state converted to bf16 storage")
    ms16, k16 = time_decode(sata, idx, st16, wl, steps, warmup, wl.seed + 30)
    kern16, fin16 = k16["decode_stream"][0], k16["decode_finish"][0]
    st16.free()
    nbytes16 = decode_bytes(wl, 2)
    ach16 = nbytes16 / (kern16 * 1e-3) / 1e9
    log("decode: window of %d steps per state update (fp32 state)" % DECODE_WINDOW)
    st = build_state(sata, idx, wl, wl.n, "f32", wl.seed)
    sata.sata_state_set_decode_window(st, DECODE_WINDOW)
    msw, kw = time_decode(sata, idx, st, wl, steps, warmup, wl.seed + 30)
    st.free()
    nread = decode_read_bytes(wl)
    read_ms, fold_ms = kw["decode_read"][0], kw["decode_fold"][0]
    ach_read = nread / (read_ms * 1e-3) / 1e9
    ach_fold = decode_bytes(wl) / (fold_ms * 1e-3) / 1e9
    nbytes = decode_bytes(wl)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    res = {
        "workload": wl.name, "value": wl.batch / (ms * 1e-3), "unit": "tokens/s",
        "ms_per_step": ms, "steps": steps, "prefix": wl.n,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "kernel": "decode_stream", "avg_launch_ms": kern_ms,
            "bytes_per_launch": nbytes, "traffic": traffic_for("decode_stream", wl.name),
        },
        "finish_ms_per_step": fin_ms,
        "gbs_whole_step": nbytes / (ms * 1e-3) / 1e9,
        "torch_streams": None,
        "f16_state": {
            "accuracy": ("binary16 words for orders >= 2, fp32 for orders 0 and 1: every step of the 1024 after "
                         "the prefix within 6e-4 of the exact Taylor output (tests: 2e-2 bar)"),
            "value": wl.batch / (msh * 1e-3), "unit": "tokens/s", "ms_per_step": msh,
            "roofline": {
                "bound": "hbm", "achieved": achh, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achh / PEAK_HBM_GBS, "kernel": "decode_stream", "avg_launch_ms": kernh,
                "bytes_per_launch": nbytesh, "traffic": traffic_for("decode_stream_f16", wl.name),
            },
            "low_orders_ms_per_step": lowh,
            "finish_ms_per_step": finh,
        },
        "bf16_state": {
            "accuracy": ("the state is rounded to bf16 after every update, and the output drifts from the exact "
                         "Taylor output past the 2e-2 bf16 bar within about 64 steps at d = 64: a bandwidth "
                         "figure for that storage, not a configuration of equal accuracy"),
            "value": wl.batch / (ms16 * 1e-3), "unit": "tokens/s", "ms_per_step": ms16,
            "roofline": {
                "bound": "hbm", "achieved": ach16, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach16 / PEAK_HBM_GBS, "kernel": "decode_stream", "avg_launch_ms": kern16,
                "bytes_per_launch": nbytes16, "traffic": traffic_for("decode_stream_bf16", wl.name),
            },
            "finish_ms_per_step": fin16,
        },
        "window": {
            "window": DECODE_WINDOW, "state": "fp32",
            "value": wl.batch / (msw * 1e-3), "unit": "tokens/s", "ms_per_step": msw,
            "roofline": {
                "bound": "hbm", "achieved": ach_read, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach_read / PEAK_HBM_GBS, "kernel": "decode_read", "avg_launch_ms": read_ms,
                "bytes_per_launch": nread, "traffic": traffic_for("decode_read", wl.name),
            },
            "fold": {"avg_launch_ms": fold_ms, "launches": kw["decode_fold"][1], "achieved_gbs": ach_fold,
                     "bytes_per_launch": decode_bytes(wl)},
            "finish_ms_per_step": kw["decode_finish"][0],
        },
    }
    ceil = stream_ceiling(decode_read_bytes(wl))
    ceil["decode_stream_vs_torch_rmw"] = achieved / ceil["torch_rmw_gbs"]
    ceil["decode_read_vs_torch_read"] = ach_read / ceil["torch_read_gbs"]
    res["torch_streams"] = ceil
    res["softmax_gap"] = decode_softmax_gap(sata, idx, wl)
    if flatness:
        flat = {}
        for prefix in (8192, 32768, 65536):
            log("decode flatness: bf16 prefill of %d tokens" % prefix)
            st = build_state(sata, idx, wl, prefix, "bf16", wl.seed + 100 + prefix)
            fms, fk = time_decode(sata, idx, st, wl, 256, 8, wl.seed + 200 + prefix)
            st.free()
            flat[str(prefix)] = {"ms_per_step": fms, "kernel_ms": fk["decode_stream"][0]}
        base = flat["8192"]["ms_per_step"]
        res["flatness"] = {"per_prefix": flat,
                           "max_rel_dev": max(abs(f["ms_per_step"] / base - 1) for f in flat.values())}
    idx.free()
    res["single_sequence"] = [decode_graph(sata, wl, d) for d in (wl.d_k, 16)]
    return res


def decode_graph(sata, wl, d: int, prefix: int = 8192, graph_steps: int = 64, reps: int = 16):
    """Small-batch decode: one sequence of the workload's heads (head size d)
    after a prefix, where the grid is small (the row-split kernels run) and,
    at small d, the host's launches set the pace.  The same steps are timed
    issued one call at a time and replayed from a HIP graph that holds
    graph_steps consecutive steps (captured once; before each replay the
    next graph_steps tokens are copied into the buffers the graph reads, and
    that copy is inside the timed region)."""
    import dataclasses
    import torch
    import synth_inputs as si
    one = dataclasses.replace(wl, batch=1, d_k=d, d_v=d)
    wl = one
    idx = sata.Index(d, d, wl.P)
    total = graph_steps * (reps + 2)
    q, k, v = si.draw_qkv_device((1, wl.heads), total, wl.d_k, wl.d_v, wl.seed + 500, "f32")
    q, k, v = (t.permute(2, 0, 1, 3).contiguous() for t in (q, k, v))     # [steps, 1, H, d]
    out = torch.empty((total, 1, wl.heads, wl.d_v), dtype=torch.float32, device="cuda")

    def eager(lo, hi):
        for t in range(lo, hi):
            sata.sata_decode_step(idx, st, q[t], k[t], v[t], out[t])

    st = build_state(sata, idx, one, prefix, "f32", wl.seed + 400)
    eager(0, graph_steps)                              # warm-up (first step allocates the workspace)
    torch.cuda.synchronize()
    lo, hi = graph_steps, graph_steps * (reps + 1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    eager(lo, hi)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / (hi - lo)
    sata.sata_profile_enable(True)
    eager(0, graph_steps)
    torch.cuda.synchronize()
    sata.sata_profile_enable(False)
    kms, kn = sata.sata_profile_query("decode_stream")
    stream_ms = kms / max(kn, 1)
    st.free()

    st = build_state(sata, idx, one, prefix, "f32", wl.seed + 400)
    eager(0, graph_steps)
    sq, sk, sv = (torch.empty((graph_steps,) + t.shape[1:], device="cuda") for t in (q, k, v))
    so = torch.empty((graph_steps,) + out.shape[1:], device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for g in range(graph_steps):
            sata.sata_decode_step(idx, st, sq[g], sk[g], sv[g], so[g])
    torch.cuda.synchronize()
    e0.record()
    for r in range(reps):
        a = graph_steps * (r + 1)
        sq.copy_(q[a:a + graph_steps]); sk.copy_(k[a:a + graph_steps]); sv.copy_(v[a:a + graph_steps])
        graph.replay()
        out[a:a + graph_steps].copy_(so)
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / (graph_steps * reps)
    st.free()
    idx.free()
    del graph, q, k, v, out, sq, sk, sv, so
    torch.cuda.empty_cache()
    nbytes = decode_bytes(wl)
    return {"workload": "1 x %d heads, d=%d, P=%d, after %d tokens" % (wl.heads, d, wl.P, prefix),
            "graph_steps": graph_steps, "eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms,
            "speedup": eager_ms / graph_ms, "stream_kernel_ms": stream_ms,
            "stream_kernel_gbs": nbytes / (stream_ms * 1e-3) / 1e9, "bytes_per_step": nbytes,
            "timing": "events on torch's stream; graph time includes the token copies in and out; "
                      "the stream kernel's time from the library's per-launch events"}


def order5_section(sata, steps: int):
    """Five orders at d = 64 (814,385 features, 212 MB of fp32 state per head):
    the prefill of prefill_d64_p5_bf16, then plain decode steps on an fp32
    state filled by a prefill of the same length."""
    import torch
    import synth_inputs as si
    wl = si.WORKLOADS["prefill_d64_p5_bf16"]
    q, k, v = si.draw_qkv_device((wl.batch, wl.heads), wl.n, wl.d_k, wl.d_v, wl.seed, wl.dtype)
    pre = time_prefill(sata, wl, q, k, v, max(3, steps // 2), 1)
    del q, k, v
    torch.cuda.empty_cache()
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = build_state(sata, idx, wl, wl.n, "bf16", wl.seed + 1)
    ms, kern = time_decode(sata, idx, st, wl, 64, 4, wl.seed + 2)
    st.free()
    idx.free()
    torch.cuda.empty_cache()
    nbytes = decode_bytes(wl)
    kms = kern["decode_stream"][0]
    ach = nbytes / (kms * 1e-3) / 1e9
    return {"prefill": pre,
            "decode": {"workload": "%d x %d heads, d=%d, P=%d, after %d tokens" % (wl.batch, wl.heads, wl.d_k, wl.P, wl.n),
                       "value": wl.batch / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
                       "stream_kernel_ms": kms, "bytes_per_step": nbytes, "achieved_gbs": ach,
                       "frac": ach / PEAK_HBM_GBS}}


def d128_section(sata):
    """Head size 128 (366,145 features at P = 4, 189 MB of fp32 state per head):
    decode for one sequence of 8 heads, plain steps from an empty state (a step's
    cost does not depend on what the state holds); the chunked prefill of
    1 x 8 x 4096 bf16 tokens, and the block path that fp32 inputs take."""
    import dataclasses
    import torch
    import synth_inputs as si
    wl = dataclasses.replace(si.WORKLOADS["decode_d64_p4_f32"], batch=1, d_k=128, d_v=128)
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    ms, kern = time_decode(sata, idx, st, wl, 64, 8, wl.seed + 3)
    nbytes = decode_bytes(wl)
    kms = kern["decode_stream"][0]
    ach = nbytes / (kms * 1e-3) / 1e9
    res = {"workload": "%d x %d heads, d=%d, P=%d" % (wl.batch, wl.heads, wl.d_k, wl.P),
           "value": wl.batch / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "stream_kernel_ms": kms,
           "bytes_per_step": nbytes, "achieved_gbs": ach, "frac": ach / PEAK_HBM_GBS}
    # prefill, bf16 inputs at P = 4: the chunked fp16-operand scan (64-token chunks)
    pwl = si.WORKLOADS["prefill_d128_p4_bf16"]
    q, k, v = si.draw_qkv_device((pwl.batch, pwl.heads), pwl.n, pwl.d_k, pwl.d_v, pwl.seed, "bf16")
    res["prefill"] = time_prefill(sata, pwl, q, k, v, 3, 1)
    res["prefill"]["workload"] = "%d x %d heads x %d tokens, d=%d, P=%d, bf16 in" % (
        pwl.batch, pwl.heads, pwl.n, pwl.d_k, pwl.P)
    # fp32 inputs take the block path (blocks of 64 tokens, each read out and folded into the
    # state in one pass: a read and a write of the state per block); one timed call
    q, k, v = (t.float() for t in (q, k, v))
    out = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    n = pwl.n
    sata.sata_state_reset(st)
    sata.sata_prefill(idx, st, q, k, v, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sata.sata_state_reset(st)
    e0.record()
    sata.sata_prefill(idx, st, q, k, v, out)
    e1.record()
    torch.cuda.synchronize()
    pms = e0.elapsed_time(e1)
    state_bytes = 4.0 * features(wl.d_k, wl.P) * (wl.d_v + 1) * wl.batch * wl.heads
    pbytes = 2 * state_bytes * ((n + 63) // 64)
    res["block_prefill_f32"] = {"workload": "%d x %d heads x %d tokens, d=%d, P=%d, fp32 in" % (
                                    wl.batch, wl.heads, n, wl.d_k, wl.P),
                                "ms_per_call": pms, "value": wl.batch * n / (pms * 1e-3), "unit": "tokens/s",
                                "state_bytes_per_call": pbytes, "achieved_gbs": pbytes / (pms * 1e-3) / 1e9,
                                "frac": pbytes / (pms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del q, k, v, out
    st.free()
    idx.free()
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ oracle on the host

def _softmax_rows(q, k, v, rows):
    """Exact causal softmax attention (fp64) of the given rows of one head:
    q, k [n, d_K], v [n, d_V] host arrays; row t attends to keys 0..t."""
    import numpy as np
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    scale = 1.0 / math.sqrt(q.shape[-1])
    out = np.empty((len(rows), v.shape[-1]))
    for i, t in enumerate(rows):
        s = k[:t + 1] @ q[t] * scale
        p = np.exp(s - s.max())
        out[i] = p @ v[:t + 1] / p.sum()
    return out


def _gap_stats(got, ref):
    """Per-row ||got - ref||_inf / ||ref||_inf: max and median."""
    import numpy as np
    e = np.max(np.abs(got - ref), axis=-1) / np.maximum(np.max(np.abs(ref), axis=-1), 1e-300)
    return {"max": float(e.max()), "median": float(np.median(e)), "rows": int(e.size)}


def prefill_softmax_gap(sata, wl, x, q, k, v, heads=(0, 7), nrows: int = 24):
    """Gap between the prefill's output (one GPU prefill of the workload, written
    in fp32 so that no output rounding adds to it) and exact softmax attention on
    the same bf16-rounded inputs, on strided rows of two heads."""
    import numpy as np
    import torch
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    out = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    sata.sata_prefill(idx, st, q, k, v, out, chunk=wl.chunk)
    torch.cuda.synchronize()
    st.free()
    idx.free()
    rows = np.unique(np.linspace(0, wl.n - 1, nrows).round().astype(np.int64))
    got, ref = [], []
    for h in heads:
        got.append(out[0, h, rows].float().cpu().numpy().astype(np.float64))
        ref.append(_softmax_rows(x.q[0, h], x.k[0, h], x.v[0, h], rows))
    res = _gap_stats(np.concatenate(got), np.concatenate(ref))
    res["sample"] = "rows %s of heads %s of %s, fp32 output" % (rows.tolist(), list(heads), wl.name)
    return res


def decode_softmax_gap(sata, idx, wl, steps: int = 48, pairs=((0, 0), (31, 7))):
    """Gap between decode outputs and exact softmax attention: a fresh state of the
    decode workload's shape, an fp32 prefill of its prefix, then `steps` decode
    steps; the inputs of two (batch, head) pairs are kept on the host and their
    outputs at every step compared with exact softmax over the whole prefix."""
    import numpy as np
    import torch
    import synth_inputs as si
    seed = wl.seed + 500
    q, k, v = si.draw_qkv_device((wl.batch, wl.heads), wl.n, wl.d_k, wl.d_v, seed, "f32")
    keep = [(q[b, h].cpu().numpy(), k[b, h].cpu().numpy(), v[b, h].cpu().numpy()) for b, h in pairs]
    st = sata.State(idx, wl.batch, wl.heads)
    out = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    sata.sata_prefill(idx, st, q, k, v, out)
    del q, k, v, out
    dq, dk, dv = si.draw_qkv_device((wl.batch, wl.heads), steps, wl.d_k, wl.d_v, seed + 1, "f32")
    dq, dk, dv = (t.permute(2, 0, 1, 3).contiguous() for t in (dq, dk, dv))     # [steps, B, H, d]
    dout = torch.empty((steps, wl.batch, wl.heads, wl.d_v), dtype=torch.float32, device="cuda")
    for t in range(steps):
        sata.sata_decode_step(idx, st, dq[t], dk[t], dv[t], dout[t])
    torch.cuda.synchronize()
    st.free()
    got, ref = [], []
    rows = np.arange(wl.n, wl.n + steps)
    for (b, h), (pq, pk, pv) in zip(pairs, keep):
        qq = np.concatenate([pq, dq[:, b, h].cpu().numpy()])
        kk = np.concatenate([pk, dk[:, b, h].cpu().numpy()])
        vv = np.concatenate([pv, dv[:, b, h].cpu().numpy()])
        got.append(dout[:, b, h].cpu().numpy().astype(np.float64))
        ref.append(_softmax_rows(qq, kk, vv, rows))
    res = _gap_stats(np.concatenate(got), np.concatenate(ref))
    res["sample"] = "decode steps %d..%d after a %d-token prefix, (batch, head) pairs %s" % (
        wl.n, wl.n + steps - 1, wl.n, [list(p) for p in pairs])
    return res


def cpu_baseline_decode(wl, budget_s: float):
    """The oracle (fp64, all host cores) on decode rows of the decode workload:
    one sequence's heads, rows right after the prefix (each row is one decode
    token of that sequence against its whole context), tokens/s = rows / time."""
    import numpy as np
    import oracle
    import synth_inputs as si
    oracle.build()
    cores = oracle.num_cpus()
    extra = 2048
    x = si.draw_qkv((1, wl.heads), wl.n + extra, wl.d_k, wl.d_v, wl.seed + 700, "f32")

    def run(r):
        rows = np.arange(wl.n, wl.n + r)
        t0 = time.perf_counter()
        oracle.taylor_attention(x.q, x.k, x.v, wl.P, rows=rows, threads=cores)
        return time.perf_counter() - t0

    t = run(4)
    r = int(min(extra, max(4, 4 * budget_s / max(t, 1e-3))))
    t = run(r)
    return {
        "value": r / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": "decode rows %d..%d (context %d+) of one sequence's %d heads of %s; %.1f s of oracle time"
                  % (wl.n, wl.n + r - 1, wl.n, wl.heads, wl.name, t),
    }


def cpu_baseline(wl, x, budget_s: float):
    """The oracle (fp64, all host cores) on uniformly strided rows of every head;
    the full-prefill time is extrapolated by n / rows (the sample's average
    context equals the full prefill's)."""
    import numpy as np
    import oracle
    oracle.build()
    cores = oracle.num_cpus()

    def run(r):
        rows = np.unique(np.linspace(0, wl.n - 1, r).round().astype(np.int64))
        t0 = time.perf_counter()
        oracle.taylor_attention(x.q, x.k, x.v, wl.P, rows=rows, threads=cores)
        return rows, time.perf_counter() - t0

    rows, t = run(16)
    r = int(min(wl.n, max(16, 16 * budget_s / max(t, 1e-3))))
    rows, t = run(r)
    per_token = t / len(rows)                       # seconds per token (all heads), average context
    return {
        "value": 1.0 / per_token, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": "%d uniformly strided rows (positions 0..%d) of all %d heads of %s; "
                  "full-prefill time extrapolated by n/rows; %.1f s of oracle time"
                  % (len(rows), wl.n - 1, wl.heads, wl.name, t),
    }


# ------------------------------------------------------------------ HBM traffic from counters

COPY_BYTES = 1 << 30
# kernel-name pattern -> (kernel, workload, source file)
TRAFFIC_KERNELS = [
    # the fp16-operand scan and the fp16-state decode (their names stay mangled in rocprofv3
    # output): D, C, positions per wave; head size, state type, storage type
    (r"scan16_kernelILi64ELi128ELi2E", "prefill_scan", "prefill_d64_p4_bf16", "sata_scan16.hip"),
    (r"scan16_kernelILi32ELi64ELi3E", "prefill_scan", "prefill_d32_p4_bf16", "sata_scan16.hip"),
    (r"scan16_kernelILi16ELi128ELi1E", "prefill_scan", "prefill_d16x64h_p4_bf16", "sata_scan16.hip"),
    (r"decode_kernel<64, float, float>", "decode_stream", "decode_d64_p4_f32", "sata_decode.hip"),
    (r"decode_rows_kernel<64, float, unsigned short, true>", "decode_stream_bf16", "decode_d64_p4_f32", "sata_decode.hip"),
    (r"decode_rows_kernelILi64EfDF16_Lb1E", "decode_stream_f16", "decode_d64_p4_f32", "sata_decode.hip"),
    (r"decode_read_kernel<64, float, float>", "decode_read", "decode_d64_p4_f32", "sata_decode.hip"),
    (r"decode_fold_kernel<64, float, float, 3, false>", "decode_fold", "decode_d64_p4_f32", "sata_decode.hip"),
]


def traffic_run():
    """One launch of every kernel whose traffic is recorded, preceded by a
    plain 1 GiB device copy that calibrates the FETCH_SIZE / WRITE_SIZE
    counters (bytes counted per byte actually moved)."""
    import torch
    import synth_inputs as si
    from constant_cost_attention_amd import sata
    sata.load()
    torch.cuda.set_device(0)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for name in ("prefill_d64_p4_bf16", "prefill_d32_p4_bf16", "prefill_d16x64h_p4_bf16"):
        wl = si.WORKLOADS[name]
        q, k, v = si.draw_qkv_device((wl.batch, wl.heads), wl.n, wl.d_k, wl.d_v, wl.seed, wl.dtype)
        idx = sata.Index(wl.d_k, wl.d_v, wl.P)
        st = sata.State(idx, wl.batch, wl.heads)
        out = torch.empty(v.shape, dtype=v.dtype, device="cuda")
        sata.sata_prefill(idx, st, q, k, v, out, chunk=wl.chunk)
        torch.cuda.synchronize()
        log("traffic run: prefill %s done" % name)
        st.free()
        idx.free()
        del q, k, v, out
        torch.cuda.empty_cache()
    wl = si.WORKLOADS["decode_d64_p4_f32"]
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = build_state(sata, idx, wl, wl.n, "f32", wl.seed)
    time_decode(sata, idx, st, wl, 2, 0, wl.seed + 30)
    log("traffic run: decode done")
    sth = sata.State(idx, wl.batch, wl.heads, dtype=torch.float16)
    sata.sata_state_convert(st, sth)
    time_decode(sata, idx, sth, wl, 2, 0, wl.seed + 30)
    log("traffic run: fp16-state decode done")
    sth.free()
    st16 = sata.State(idx, wl.batch, wl.heads, dtype=torch.bfloat16)
    sata.sata_state_convert(st, st16)
    st.free()
    time_decode(sata, idx, st16, wl, 2, 0, wl.seed + 30)
    log("traffic run: bf16-state decode done")
    st16.free()
    st = build_state(sata, idx, wl, wl.n, "f32", wl.seed)
    sata.sata_state_set_decode_window(st, 2)
    time_decode(sata, idx, st, wl, 2, 0, wl.seed + 30)      # one read step, one fold (of two tokens)
    log("traffic run: windowed decode done")
    st.free()
    idx.free()


def _counter_means(path: str, counter: str):
    """Per-dispatch counter values (KiB) from a rocprofv3 counter_collection CSV,
    summed over the counter's instances, grouped by kernel name."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            key = (row["Dispatch_Id"], row["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    by_name = {}
    for (_, name), val in per.items():
        by_name.setdefault(name, []).append(val)
    return by_name


def write_traffic(fetch_csv: str, write_csv: str):
    import re
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    copies = [n for n in fetch if "copy" in n.lower() and "sata::" not in n]
    if not copies:
        raise SystemExit("no copy kernel among: %s" % sorted(fetch))
    copy_name = max(copies, key=lambda n: max(fetch[n]))
    kib = COPY_BYTES / 1024.0
    f_fetch = kib / max(fetch[copy_name])
    f_write = kib / max(write[copy_name])
    out = {"_calibration": {"copy_kernel": copy_name, "copy_bytes_each_way": COPY_BYTES,
                            "fetch_kib_read": max(fetch[copy_name]), "write_kib_read": max(write[copy_name]),
                            "fetch_factor": f_fetch, "write_factor": f_write}}
    for pat, kernel, workload, source in TRAFFIC_KERNELS:
        names = [n for n in fetch if re.search(pat, n)]
        if len(names) != 1:
            raise SystemExit("pattern %s matched %s" % (pat, names))
        n = names[0]
        fk = sum(fetch[n]) / len(fetch[n])
        wk = sum(write[n]) / len(write[n])
        out.setdefault(kernel, {})[workload] = {
            "source": source, "source_sha256": source_sha(source), "kernel_name": n,
            "dispatches": len(fetch[n]), "fetch_kib": fk, "write_kib": wk,
            "bytes_per_launch": (fk * f_fetch + wk * f_write) * 1024.0,
        }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out, indent=1, sort_keys=True))


# ------------------------------------------------------------------ main

def main():
    args = parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU; --gpus %d (WORLD_SIZE=%d) is not supported: "
              "multi-GPU execution is not implemented" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.traffic_run:
        traffic_run()
        return
    import torch
    import synth_inputs as si
    from constant_cost_attention_amd import sata
    sata.load()
    torch.cuda.set_device(0)
    if args.tile_sweep:
        print(json.dumps({"tile_sweep": tile_sweep(sata)}))
        return
    if args.backward_only:
        out = []
        for name in BACKWARD_WORKLOADS:
            bw = time_backward(sata, si.WORKLOADS[name], args.steps)
            log("backward %s: %.2f ms per call" % (name, bw["ms_per_call"]))
            out.append(bw)
        print(json.dumps({"backward": out}))
        return

    wl = si.WORKLOADS[METRIC_WORKLOAD]
    log("drawing %s inputs" % wl.name)
    x = wl.draw()
    q, k, v = upload(x)
    log("prefill %s: %d warmup + %d timed steps" % (wl.name, args.warmup, args.steps))
    pre = time_prefill(sata, wl, q, k, v, args.steps, args.warmup)
    log("prefill: %.3f ms/step, %.3e tok/s, scan %.1f TFLOP/s (%.1f%% of peak)"
        % (pre["ms_per_step"], pre["value"], pre["roofline"]["achieved"], 100 * pre["roofline"]["frac"]))
    gap = prefill_softmax_gap(sata, wl, x, q, k, v)
    log("prefill vs exact softmax: max %.3e, median %.3e over %d rows" % (gap["max"], gap["median"], gap["rows"]))
    del q, k, v
    ceil = {"f16_16x16x32_tflops": sata.sata_measure_mfma_loop(False),
            "bf16_16x16x32_tflops": sata.sata_measure_mfma_loop(True)}
    ceil["method"] = ("a loop of 16 independent in-place MFMA chains per wavefront, two wavefronts per SIMD on "
                      "every compute unit, nothing else in the loop (the scan issues the fp16 instruction)")
    pre["roofline"]["mfma_loop_ceiling"] = ceil
    pre["roofline"]["frac_of_ceiling"] = pre["roofline"]["achieved"] / ceil["f16_16x16x32_tflops"]
    log("MFMA loop ceiling: fp16 %.1f, bf16 %.1f TFLOP/s (scan at %.1f%% of the fp16 loop)"
        % (ceil["f16_16x16x32_tflops"], ceil["bf16_16x16x32_tflops"], 100 * pre["roofline"]["frac_of_ceiling"]))
    torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": pre["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads, "seq_len": wl.n,
                   "d_k": wl.d_k, "d_v": wl.d_v, "P": wl.P, "chunk": wl.chunk,
                   "inputs": "bf16 q/k/v, fp32 state", "parallelism": "single GPU"},
        "roofline": pre["roofline"],
        "prefill": {k2: pre[k2] for k2 in ("tflops_whole_call", "combine_ms_per_step")},
        "softmax_gap": gap,
    }

    if not args.no_decode:
        dwl = si.WORKLOADS["decode_d64_p4_f32"]
        dec = decode_section(sata, dwl, args.decode_steps, 8, not args.no_flatness)
        log("decode: %.3f ms/step, %.3e tok/s, stream %.0f GB/s (%.1f%% of peak)"
            % (dec["ms_per_step"], dec["value"], dec["roofline"]["achieved"], 100 * dec["roofline"]["frac"]))
        h16 = dec["f16_state"]
        log("decode, fp16 state: %.3f ms/step, %.3e tok/s, stream %.0f GB/s (%.1f%% of peak), fp32 orders %.3f ms"
            % (h16["ms_per_step"], h16["value"], h16["roofline"]["achieved"], 100 * h16["roofline"]["frac"],
               h16["low_orders_ms_per_step"]))
        b16 = dec["bf16_state"]
        log("decode, bf16 state: %.3f ms/step, %.3e tok/s, stream %.0f GB/s (%.1f%% of peak)"
            % (b16["ms_per_step"], b16["value"], b16["roofline"]["achieved"], 100 * b16["roofline"]["frac"]))
        c = dec["torch_streams"]
        log("decode beside torch streams: in-place RMW %.0f GB/s (decode kernel at %.2fx), row-sum read %.0f GB/s "
            "(read kernel at %.2fx)" % (c["torch_rmw_gbs"], c["decode_stream_vs_torch_rmw"], c["torch_read_gbs"],
                                        c["decode_read_vs_torch_read"]))
        g = dec["softmax_gap"]
        log("decode vs exact softmax: max %.3e, median %.3e over %d rows" % (g["max"], g["median"], g["rows"]))
        dw = dec["window"]
        log("decode, window %d: %.3f ms/step, %.3e tok/s, read %.3f ms at %.0f GB/s (%.1f%% of peak), "
            "fold %.3f ms at %.0f GB/s"
            % (dw["window"], dw["ms_per_step"], dw["value"], dw["roofline"]["avg_launch_ms"],
               dw["roofline"]["achieved"], 100 * dw["roofline"]["frac"], dw["fold"]["avg_launch_ms"],
               dw["fold"]["achieved_gbs"]))
        for gr in dec["single_sequence"]:
            log("decode, %s: %.1f us/step issued call by call, %.1f us/step replayed from a graph of %d steps; "
                "stream kernel %.1f us at %.0f GB/s"
                % (gr["workload"], 1e3 * gr["eager_ms_per_step"], 1e3 * gr["graph_ms_per_step"], gr["graph_steps"],
                   1e3 * gr["stream_kernel_ms"], gr["stream_kernel_gbs"]))
        result["decode"] = dec
        torch.cuda.empty_cache()

    if not args.no_extra:
        extra = []
        for name in ("prefill_d32_p4_bf16", "prefill_d16x64h_p4_bf16", "prefill_d16_p4_f32"):
            ewl = si.WORKLOADS[name]
            eq, ek, ev = si.draw_qkv_device((ewl.batch, ewl.heads), ewl.n, ewl.d_k, ewl.d_v, ewl.seed, ewl.dtype)
            r = time_prefill(sata, ewl, eq, ek, ev, max(3, args.steps // 2), 1)
            log("extra %s: %.3f ms/step, %.3e tok/s, %.1f%% of peak"
                % (name, r["ms_per_step"], r["value"], 100 * r["roofline"]["frac"]))
            extra.append(r)
            del eq, ek, ev
            torch.cuda.empty_cache()
        result["extra"] = extra
        o5 = order5_section(sata, args.steps)
        log("order 5, %s: %.3f ms/step, %.3e tok/s, %.1f%% of peak; decode %s: %.3f ms/step, stream %.0f GB/s "
            "(%.1f%% of peak)" % (o5["prefill"]["workload"], o5["prefill"]["ms_per_step"], o5["prefill"]["value"],
                                  100 * o5["prefill"]["roofline"]["frac"], o5["decode"]["workload"],
                                  o5["decode"]["ms_per_step"], o5["decode"]["achieved_gbs"], 100 * o5["decode"]["frac"]))
        result["order5"] = o5
        dd = d128_section(sata)
        log("decode, %s: %.3f ms/step, stream %.0f GB/s (%.1f%% of peak)" % (
            dd["workload"], dd["ms_per_step"], dd["achieved_gbs"], 100 * dd["frac"]))
        log("chunked prefill %s: %.2f ms, %.3e tok/s, scan %.1f%% of peak; block prefill %s: %.2f ms, %.3e tok/s"
            % (dd["prefill"]["workload"], dd["prefill"]["ms_per_step"], dd["prefill"]["value"],
               100 * dd["prefill"]["roofline"]["frac"], dd["block_prefill_f32"]["workload"],
               dd["block_prefill_f32"]["ms_per_call"], dd["block_prefill_f32"]["value"]))
        result["d128"] = dd

    if not args.no_backward:
        bwd = []
        for name in BACKWARD_WORKLOADS:
            bw = time_backward(sata, si.WORKLOADS[name], 2)
            if name == METRIC_WORKLOAD:
                bw["vs_forward_call"] = bw["ms_per_call"] / result["ms_per_step"]
            log("backward %s: %.2f ms per call, %.3e tok/s, %.1f TFLOP/s algorithmic%s"
                % (name, bw["ms_per_call"], bw["value"], bw["algorithmic_tflops"],
                   ", %.1fx the forward call" % bw["vs_forward_call"] if "vs_forward_call" in bw else ""))
            bwd.append(bw)
        result["backward"] = bwd

    if not args.no_cpu:
        log("cpu baseline: oracle on the host (budget %.0f s)" % args.cpu_budget)
        result["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_budget)
        log("cpu baseline: %.3e tok/s on %d cores" % (result["cpu_baseline"]["value"],
                                                      result["cpu_baseline"]["cores"]))
        if "decode" in result:
            dwl = si.WORKLOADS["decode_d64_p4_f32"]
            result["decode"]["cpu_baseline"] = cpu_baseline_decode(dwl, args.cpu_budget / 2)
            log("cpu baseline, decode: %.3e tok/s on %d cores" % (result["decode"]["cpu_baseline"]["value"],
                                                                   result["decode"]["cpu_baseline"]["cores"]))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
