"""Seeded synthetic inputs for SATA attention.

This module is the only code shared by the HIP path's tests/benchmark and the
oracle: it draws inputs and rounds them to the storage dtype, and holds none
of the attention arithmetic.

Recipe (the workloads the method is measured on are synthetic):
  1. numpy.random.Generator(PCG64(seed)); draw q, then k, then v, each as a
     full float64 array of standard normals, in that order.
  2. q and k rows are L2-normalised and scaled by d_K**0.25, so that the
     scaled logit q.k/sqrt(d_K) lies in [-1, 1].
  3. v stays N(0, 1).
  4. All three are rounded to the storage dtype: float32 (round to nearest),
     or bfloat16 (round to nearest even).  The rounded array is what both the
     GPU and the oracle consume (the oracle widens it exactly).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20260205


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits.
    NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((x.view(np.uint32)[nan] >> 16) | 0x0040).astype(np.uint16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32, exactly."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class QKV:
    """One seeded draw.  ``q, k, v`` are float32 arrays holding the exact values
    consumed by both sides; for bf16 inputs ``q_bits`` etc. hold the uint16
    storage the GPU receives."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str
    bits: dict = field(default_factory=dict)

    def storage(self, name: str) -> np.ndarray:
        """The array in its storage dtype (float32, or uint16 bf16 bits)."""
        if self.dtype == "bf16":
            return self.bits[name]
        return getattr(self, name)


def draw_qkv(lead: tuple, n: int, d_k: int, d_v: int, seed: int, dtype: str = "f32") -> QKV:
    """Draw q, k: [*lead, n, d_K], v: [*lead, n, d_V] per the recipe above."""
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    rng = np.random.Generator(np.random.PCG64(seed))
    shape_k = tuple(lead) + (n, d_k)
    shape_v = tuple(lead) + (n, d_v)
    arrays = {}
    for name, shp in (("q", shape_k), ("k", shape_k), ("v", shape_v)):
        g = rng.standard_normal(shp)                       # float64
        if name != "v":
            nrm = np.sqrt(np.sum(g * g, axis=-1, keepdims=True))
            nrm[nrm == 0] = 1.0
            g = g / nrm * (float(d_k) ** 0.25)
        arrays[name] = g.astype(np.float32)
        del g
    if dtype == "bf16":
        bits = {name: bf16_bits(a) for name, a in arrays.items()}
        vals = {name: bf16_to_f32(b) for name, b in bits.items()}
        return QKV(vals["q"], vals["k"], vals["v"], "bf16", bits)
    return QKV(arrays["q"], arrays["k"], arrays["v"], "f32")


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload: batch x heads x n tokens, head dims, orders P,
    input dtype, chunk length, seed."""
    name: str
    batch: int
    heads: int
    n: int
    d_k: int
    d_v: int
    P: int
    dtype: str
    chunk: int
    seed: int
    decode_steps: int = 0

    def draw(self, n: int | None = None) -> QKV:
        return draw_qkv((self.batch, self.heads), self.n if n is None else n,
                        self.d_k, self.d_v, self.seed, self.dtype)

    def draw_decode(self, steps: int | None = None) -> QKV:
        """Fresh per-step decode inputs [B, H, steps, d] with their own seed."""
        s = self.decode_steps if steps is None else steps
        return draw_qkv((self.batch, self.heads), s, self.d_k, self.d_v, SEED_BASE + 30, "f32")


# The measured workloads.  Sizes, orders and dtypes as the method's cost
# figures and the stated targets use them (d_K = d_V in every case).
WORKLOADS = {
    "tiny_d8_p3": Workload("tiny_d8_p3", 1, 1, 256, 8, 8, 3, "f32", 64, SEED_BASE + 0),
    "prefill_d16_p4_f32": Workload("prefill_d16_p4_f32", 1, 8, 4096, 16, 16, 4, "f32", 128, SEED_BASE + 1),
    "prefill_d32_p4_bf16": Workload("prefill_d32_p4_bf16", 2, 16, 16384, 32, 32, 4, "bf16", 64, SEED_BASE + 2),
    "decode_d64_p4_f32": Workload("decode_d64_p4_f32", 32, 8, 8192, 64, 64, 4, "f32", 128, SEED_BASE + 3,
                                  decode_steps=1024),
    "prefill_d64_p4_bf16": Workload("prefill_d64_p4_bf16", 1, 8, 65536, 64, 64, 4, "bf16", 128, SEED_BASE + 4),
    "prefill_d16x64h_p4_bf16": Workload("prefill_d16x64h_p4_bf16", 1, 64, 131072, 16, 16, 4, "bf16", 128,
                                        SEED_BASE + 5),
    # five orders (814,385 features, 212 MB of fp32 state per head at d = 64)
    "prefill_d64_p5_bf16": Workload("prefill_d64_p5_bf16", 1, 8, 8192, 64, 64, 5, "bf16", 128, SEED_BASE + 6),
    # head size 128 (366,145 features, 189 MB of fp32 state per head), 64-token chunks
    "prefill_d128_p4_bf16": Workload("prefill_d128_p4_bf16", 1, 8, 4096, 128, 128, 4, "bf16", 64, SEED_BASE + 7),
}


def draw_qkv_device(lead: tuple, n: int, d_k: int, d_v: int, seed: int, dtype: str = "f32",
                    device: str = "cuda"):
    """Same recipe drawn on the GPU with a seeded torch generator (timing-only
    inputs: long prefixes whose values no parity check reads).  Returns torch
    tensors (q, k, v) in float32 or bfloat16."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = []
    for name, dd in (("q", d_k), ("k", d_k), ("v", d_v)):
        g = torch.randn(tuple(lead) + (n, dd), generator=gen, device=device, dtype=torch.float32)
        if name != "v":
            g = g / g.norm(dim=-1, keepdim=True).clamp_min(1e-30) * (float(d_k) ** 0.25)
        out.append(g.to(tdt).contiguous())
    return tuple(out)
