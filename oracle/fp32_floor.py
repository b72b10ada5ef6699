"""The error that fp32 state accumulation carries by itself, at the lengths of
the fp32 workloads (TEST INFRASTRUCTURE / report only; calls nothing but the
oracle and the seeded input generators).

For one head of each case, O7 (the recurrent form with its state and
arithmetic in float) against O1 (the exact quadratic definition, fp64), on the
workload's own seeded inputs:
  prefill_d16_p4_f32   every row of n = 4096 tokens (d = 16, P = 4);
  decode_d64_p4_f32    the 1024 decode rows after the 8192-token prefix
                       (d = 64, P = 4), the prefix rows on a stride.
The metric is the per-row normwise error max_c |o - o_ref| / max_c |o_ref|,
reported as its maximum and mean over the rows and at the last row.  This is
what an implementation that keeps the state in fp32 and sums token by token
gets without any other error source: the floor under the fp32 parity bar.
O7 runs on one thread per head; the d = 64 case takes a few minutes.

Usage: python -m oracle.fp32_floor [--skip-d64]
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _rowerr(a, ref):
    return np.max(np.abs(a - ref), axis=-1) / np.max(np.abs(ref), axis=-1)


def floor_case(name, q, k, v, P, rows):
    import oracle
    t0 = time.time()
    o7 = oracle.recurrent_attention_f32(q, k, v, P)[..., rows, :]
    o1 = oracle.taylor_attention(q, k, v, P, rows=rows)
    e = _rowerr(o7, o1).reshape(-1)
    print("%-22s rows %5d  max %.2e  mean %.2e  last %.2e  (%.0f s)" %
          (name, len(rows), e.max(), e.mean(), e[-1], time.time() - t0), flush=True)
    return e


def main():
    import oracle
    import synth_inputs as si
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--skip-d64", action="store_true")
    args = ap.parse_args()
    oracle.build()
    wl = si.WORKLOADS["prefill_d16_p4_f32"]
    x = wl.draw()
    sl = lambda a: np.ascontiguousarray(a[:1, :1])
    floor_case(wl.name, sl(x.q), sl(x.k), sl(x.v), wl.P, np.arange(wl.n))
    if not args.skip_d64:
        wl = si.WORKLOADS["decode_d64_p4_f32"]
        pre = wl.draw()
        dec = wl.draw_decode(1024)
        cat = lambda a, b: np.concatenate([a[:1, :1], b[:1, :1]], axis=2)
        q, k, v = cat(pre.q, dec.q), cat(pre.k, dec.k), cat(pre.v, dec.v)
        floor_case(wl.name + " decode", q, k, v, wl.P, np.arange(wl.n, wl.n + 1024))
        floor_case(wl.name + " prefix", q, k, v, wl.P, np.arange(0, wl.n, 64))


if __name__ == "__main__":
    main()
