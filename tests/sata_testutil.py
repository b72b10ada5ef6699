"""Helpers shared by the GPU parity tests: device upload of seeded inputs, the
error metric, row sampling and one-call wrappers around the binding."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth_inputs as si

TOL_F32 = 1e-5      # max over rows of |o - o_ref|_inf / |o_ref|_inf, fp32 inputs
TOL_BF16 = 2e-2     # same metric, bf16 inputs (oracle consumes the bf16-rounded values)


def say(msg: str):
    """Name the case before any GPU work, flushed, so a fault can be attributed."""
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(o, ref) -> float:
    """max over rows of ||o_i - ref_i||_inf / ||ref_i||_inf (per-row normwise)."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(o - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.max(num / np.maximum(den, 1e-300)))


def dev(qkv: si.QKV, name: str) -> torch.Tensor:
    """Upload one array in its storage dtype (float32, or bf16 from its bits)."""
    a = qkv.storage(name)
    if qkv.dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def dev_all(qkv: si.QKV):
    return dev(qkv, "q"), dev(qkv, "k"), dev(qkv, "v")


def sample_rows(n: int, chunk: int, extra: int, seed: int) -> np.ndarray:
    """Rows of the first and last chunk plus `extra` seeded uniform rows."""
    rows = set(range(min(n, chunk)))
    rows |= set(range(max(0, n - chunk), n))
    rng = np.random.default_rng(seed)
    rows |= set(rng.integers(0, n, size=extra).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def prefill(index, state, q, k, v, chunk=0, out_dtype=torch.float32):
    from constant_cost_attention_amd import sata
    out = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    sata.sata_prefill(index, state, q, k, v, out, chunk=chunk)
    return out


def decode(index, state, q, k, v, out_dtype=torch.float32):
    from constant_cost_attention_amd import sata
    out = torch.empty(v.shape, dtype=out_dtype, device=v.device)
    sata.sata_decode_step(index, state, q, k, v, out)
    return out
