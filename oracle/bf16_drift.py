"""Drift of a 16-bit decode state from the exact result (TEST INFRASTRUCTURE
/ report only; calls nothing but the oracle and the seeded input generators).

The page suggests 16-bit storage to halve the state's bandwidth [hotdry,
"Hardware optimisation paths and current limits"].  Here the prefix of a
workload is summed exactly and rounded to bf16 once, then T decode steps run on
the bf16-stored state (O8: add exactly, read out, store rounded to nearest
even), and each step's output is compared with the exact Taylor attention
(O1) of the same row.  For scale, the same rows' gap between Taylor and exact
softmax attention (O2) is printed: the error the method itself carries.

Columns: the workload, heads used, prefix length n0, then for each checkpoint
t the largest row error over steps 1..t (max over rows of
||o - o_exact||_inf / ||o_exact||_inf), then the Taylor-vs-softmax gap on
the same rows.

With --f16 L the state is fp16 with the orders below L kept in fp32 (O8's
fp16 form) instead of bf16.

Usage: python -m oracle.bf16_drift [--steps 256] [--f16 L]
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CHECKPOINTS = (1, 4, 16, 64, 256, 1024)


def _row_err(a, ref):
    return np.max(np.abs(a - ref), axis=-1) / np.max(np.abs(ref), axis=-1)


def drift(name: str, heads: int, steps: int, threads: int, f16_low: int = -1):
    import oracle
    import synth_inputs as si
    wl = si.WORKLOADS[name]
    pre = wl.draw()
    dec = si.draw_qkv((wl.batch, wl.heads), steps, wl.d_k, wl.d_v, wl.seed + 7919, "f32")
    pick = lambda a: a.reshape((-1,) + a.shape[-2:])[:heads]
    q = np.concatenate([pick(pre.q), pick(dec.q)], axis=1)
    k = np.concatenate([pick(pre.k), pick(dec.k)], axis=1)
    v = np.concatenate([pick(pre.v), pick(dec.v)], axis=1)
    rows = np.arange(wl.n, wl.n + steps, dtype=np.int64)
    if f16_low >= 0:
        o16 = oracle.f16_state_decode(q, k, v, wl.P, wl.n, low_orders=f16_low)
    else:
        o16 = oracle.bf16_state_decode(q, k, v, wl.P, wl.n)
    exact = oracle.taylor_attention(q, k, v, wl.P, rows=rows, threads=threads)
    soft = oracle.softmax_attention(q, k, v, rows=rows, threads=threads)
    e = _row_err(o16, exact).max(axis=0)             # per step, worst head
    running = np.maximum.accumulate(e)
    gap = float(_row_err(exact, soft).max())
    return wl, {t: float(running[t - 1]) for t in CHECKPOINTS if t <= steps}, gap


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--f16", type=int, default=-1, help="fp16 state with the orders below this in fp32")
    args = ap.parse_args()
    import oracle
    oracle.build()
    threads = oracle.num_cpus()
    cps = [t for t in CHECKPOINTS if t <= max(args.steps, 1024)]
    print("| workload | heads | n0 | " + " | ".join("t<=%d" % t for t in cps) + " | Taylor vs softmax |")
    print("|---|---|---|" + "---|" * len(cps) + "---|")
    for name, heads, steps in (("tiny_d8_p3", 1, 1024), ("prefill_d16_p4_f32", 2, 1024),
                               ("prefill_d32_p4_bf16", 1, args.steps), ("decode_d64_p4_f32", 1, args.steps)):
        wl, d, gap = drift(name, heads, steps, threads, args.f16)
        cells = ["%.2e" % d[t] if t in d else "" for t in cps]
        print("| %s | %d | %d | %s | %.2e |" % (name, heads, wl.n, " | ".join(cells), gap), flush=True)


if __name__ == "__main__":
    main()
