"""Gap between the truncated-Taylor attention and exact softmax attention on the
synthetic workloads (TEST INFRASTRUCTURE / report only; calls nothing but the
oracle and the seeded input generators).

For each workload, on uniformly strided rows of (up to) its first 8 heads:
  taylor_vs_softmax  max and mean over rows of ||o_T - o_S||_inf / ||o_S||_inf
                     with o_T the P-term Taylor attention (O1) and o_S exact
                     softmax attention (O2), both fp64 on the same inputs;
  fp16_softmax       the same metric for softmax evaluated on fp16-rounded
                     q, k, v with its output rounded to fp16, against o_S: the
                     error of a plain fp16 evaluation, the yardstick the page
                     compares P = 4 with [hotdry, "Precision/efficiency
                     trade-off"];
  bound              the per-weight Lagrange remainder bound e^|x| |x|^P / P!
                     relative to e^x, at |x| <= 1: e^2 / P!.

Usage: python -m oracle.softmax_gap [--rows 64]
"""
from __future__ import annotations

import argparse
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _rowwise(a, ref):
    err = np.max(np.abs(a - ref), axis=-1) / np.max(np.abs(ref), axis=-1)
    return float(err.max()), float(err.mean())


def gap(wl, nrows: int, threads: int):
    import oracle
    import synth_inputs as si
    x = wl.draw()
    heads = min(8, wl.batch * wl.heads)
    shape = lambda a: a.reshape((-1,) + a.shape[-2:])[:heads]
    q, k, v = shape(x.q), shape(x.k), shape(x.v)
    rows = np.unique(np.linspace(0, wl.n - 1, nrows).round().astype(np.int64))
    o_t = oracle.taylor_attention(q, k, v, wl.P, rows=rows, threads=threads)
    o_s = oracle.softmax_attention(q, k, v, rows=rows, threads=threads)
    h16 = lambda a: a.astype(np.float16).astype(np.float32)
    o_h = oracle.softmax_attention(h16(q), h16(k), h16(v), rows=rows, threads=threads)
    o_h = o_h.astype(np.float16).astype(np.float64)
    del si
    return {
        "workload": wl.name, "heads": heads, "rows": len(rows), "P": wl.P,
        "taylor_vs_softmax": _rowwise(o_t, o_s),
        "fp16_softmax": _rowwise(o_h, o_s),
        "bound": math.e ** 2 / math.factorial(wl.P),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=64)
    args = ap.parse_args()
    import oracle
    import synth_inputs as si
    oracle.build()
    threads = oracle.num_cpus()
    print("| workload | P | heads x rows | Taylor vs softmax: max | mean | fp16 softmax vs softmax: max | mean | e^2/P! |")
    print("|---|---|---|---|---|---|---|---|")
    for name in ("tiny_d8_p3", "prefill_d16_p4_f32", "prefill_d32_p4_bf16", "decode_d64_p4_f32",
                 "prefill_d64_p4_bf16", "prefill_d16x64h_p4_bf16"):
        r = gap(si.WORKLOADS[name], args.rows, threads)
        print("| %s | %d | %d x %d | %.3e | %.3e | %.3e | %.3e | %.3e |" % (
            r["workload"], r["P"], r["heads"], r["rows"], *r["taylor_vs_softmax"], *r["fp16_softmax"], r["bound"]),
            flush=True)


if __name__ == "__main__":
    main()
