"""SATA oracle: TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 CPU implementation of symmetry-aware Taylor approximation
(SATA) attention, used to check the HIP library.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with ``constant_cost_attention_amd`` and never
imports it; the product path never imports this package.

Sources, cited by page and section:

* [hotdry] blog.hotdry.top, "Symmetry-aware Taylor approximation attention:
  engineering a constant per-token cost" (2026-02-05): sections "Scale
  bottleneck of conventional self-attention", "Core insight of symmetric
  tensor decomposition", "Engineering realisation of the constant compute
  cost", "Precision/efficiency trade-off".
* [mokono] www.mokono.cn attention-variants survey, standard attention:
  the (batch, heads, seq, dim) layout and the 1/sqrt(d) logit scale.

Functions (what pins each one is listed in the tests and in the design notes):

* ``taylor_attention``   O1, quadratic causal Taylor-weighted attention.
* ``softmax_attention``  O2, exact causal softmax attention (gap report only).
* ``basis_bruteforce``   O3, sorted-tuple groups of all d^p ordered tuples.
* ``phi``                O4, symmetric feature map from the O3 groups.
* ``recurrent_attention`` O5, the constant-size state form (tiny inputs).
* ``recurrent_attention_f32`` O7, O5 carried out in float (diagnostic).
* ``round_bf16``         O8a, round to nearest bfloat16, ties to even.
* ``bf16_state_decode``  O8, decode steps on a state stored in bf16.
* ``round_f16``          O8b, round to nearest IEEE binary16, ties to even.
* ``f16_state_decode``   O8 for an fp16 state whose lowest orders are fp32.
* ``taylor_attention_grad`` O9, gradients of O1 (fp64 autograd of the
  quadratic form, plain PyTorch CPU ops).
* ``basis_size``, ``state_size``, ``flops_per_token`` O6, the closed forms the
  page prints, in exact integers.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sata_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
            "-std=c11", _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB_PATH)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64, cint = ctypes.c_int64, ctypes.c_int
    lib.orc_num_cpus.restype = cint
    lib.orc_taylor_attention.argtypes = [f32p, f32p, f32p, f64p, i64, i64, cint, cint, cint, i64p, i64, cint]
    lib.orc_taylor_attention.restype = cint
    lib.orc_softmax_attention.argtypes = [f32p, f32p, f32p, f64p, i64, i64, cint, cint, i64p, i64, cint]
    lib.orc_softmax_attention.restype = cint
    lib.orc_basis_bruteforce.argtypes = [cint, cint, i32p, i64p, i64]
    lib.orc_basis_bruteforce.restype = i64
    lib.orc_phi.argtypes = [f64p, cint, cint, f64p, i64]
    lib.orc_phi.restype = i64
    lib.orc_round_bf16_array.argtypes = [f64p, f64p, i64]
    lib.orc_round_bf16_array.restype = None
    lib.orc_bf16_state_decode.argtypes = [f32p, f32p, f32p, f64p, i64, i64, i64, cint, cint, cint, cint, cint]
    lib.orc_bf16_state_decode.restype = cint
    lib.orc_round_f16_array.argtypes = [f64p, f64p, i64]
    lib.orc_round_f16_array.restype = None
    lib.orc_f16_state_decode.argtypes = [f32p, f32p, f32p, f64p, i64, i64, i64, cint, cint, cint, i64, cint]
    lib.orc_f16_state_decode.restype = cint
    for name in ("orc_recurrent_attention", "orc_recurrent_attention_f32"):
        fn = getattr(lib, name)
        fn.argtypes = [f32p, f32p, f32p, f64p, i64, i64, cint, cint, cint]
        fn.restype = cint
    _lib = lib
    return lib


def num_cpus() -> int:
    """Threads the oracle uses by default (the process's CPU affinity count)."""
    return int(_load().orc_num_cpus())


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _heads(q, k, v):
    """Flatten leading (batch, heads) dims: [..., n, d] -> [bh, n, d]."""
    if q.ndim < 2:
        raise ValueError("q must be [..., n, d_K]")
    lead = q.shape[:-2]
    n, dk = q.shape[-2:]
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:-1] != q.shape[:-1]:
        raise ValueError("q, k, v shapes disagree: %s %s %s" % (q.shape, k.shape, v.shape))
    bh = int(np.prod(lead)) if lead else 1
    return lead, bh, n, dk, dv


def _rows_arg(rows, n):
    if rows is None:
        return None, None, n
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.ndim != 1 or (r.size and (r.min() < 0 or r.max() >= n)):
        raise ValueError("rows must be a 1-D list of indices in [0, n)")
    return r, r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), r.size


def taylor_attention(q, k, v, P: int, rows=None, threads: int = 0) -> np.ndarray:
    """O1: o_i = sum_{j<=i} w(x_ij) v_j / sum_{j<=i} w(x_ij), w(x) = sum_{p<P} x^p/p!,
    x_ij = q_i.k_j/sqrt(d_K)  [hotdry, "Core insight of symmetric tensor
    decomposition" (the truncated exp kernel) and "Engineering realisation of
    the constant compute cost" (the normalising "+1" column)].

    q, k: [..., n, d_K]; v: [..., n, d_V] (any float dtype; converted to fp32,
    which must represent them exactly).  Returns float64 [..., len(rows) or n, d_V].
    """
    lead, bh, n, dk, dv = _heads(np.asarray(q), np.asarray(k), np.asarray(v))
    q32, qp = _f32(q)
    k32, kp = _f32(k)
    v32, vp = _f32(v)
    r, rp, nr = _rows_arg(rows, n)
    out = np.empty((bh, nr, dv), dtype=np.float64)
    rc = _load().orc_taylor_attention(qp, kp, vp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                      bh, n, dk, dv, int(P), rp, nr, int(threads))
    if rc:
        raise ValueError("orc_taylor_attention rejected its arguments (rc=%d)" % rc)
    return out.reshape(tuple(lead) + (nr, dv))


def softmax_attention(q, k, v, rows=None, threads: int = 0) -> np.ndarray:
    """O2: exact causal softmax attention with the same layout and scale
    [hotdry, "Scale bottleneck of conventional self-attention"]."""
    lead, bh, n, dk, dv = _heads(np.asarray(q), np.asarray(k), np.asarray(v))
    q32, qp = _f32(q)
    k32, kp = _f32(k)
    v32, vp = _f32(v)
    r, rp, nr = _rows_arg(rows, n)
    out = np.empty((bh, nr, dv), dtype=np.float64)
    rc = _load().orc_softmax_attention(qp, kp, vp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                       bh, n, dk, dv, rp, nr, int(threads))
    if rc:
        raise ValueError("orc_softmax_attention rejected its arguments (rc=%d)" % rc)
    return out.reshape(tuple(lead) + (nr, dv))


def basis_bruteforce(d: int, p: int):
    """O3: (tuples [g, p] int32 in lexicographic order, counts [g] int64) of the
    sorted-tuple groups of all d^p ordered index tuples
    [hotdry, "Core insight of symmetric tensor decomposition"]."""
    lib = _load()
    g = lib.orc_basis_bruteforce(int(d), int(p), None, None, 0)
    if g < 0:
        raise ValueError("brute force limit exceeded or bad arguments (d=%d, p=%d)" % (d, p))
    tup = np.zeros((g, max(p, 1)), dtype=np.int32)
    cnt = np.zeros((g,), dtype=np.int64)
    lib.orc_basis_bruteforce(int(d), int(p), tup.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                             cnt.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), g)
    return tup[:, :p], cnt


def phi(x, p: int) -> np.ndarray:
    """O4: symmetric feature map phi_p(x)_t = sqrt(count_t) prod_r x[t_r] over the
    brute-force groups, so phi_p(q).phi_p(k) = (q.k)^p."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    d = x.shape[0]
    lib = _load()
    g = lib.orc_basis_bruteforce(d, int(p), None, None, 0)
    out = np.empty((g,), dtype=np.float64)
    rc = lib.orc_phi(x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), d, int(p),
                     out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), g)
    if rc < 0:
        raise ValueError("orc_phi failed")
    return out


def _recurrent(name, q, k, v, P):
    lead, bh, n, dk, dv = _heads(np.asarray(q), np.asarray(k), np.asarray(v))
    q32, qp = _f32(q)
    k32, kp = _f32(k)
    v32, vp = _f32(v)
    out = np.empty((bh, n, dv), dtype=np.float64)
    rc = getattr(_load(), name)(qp, kp, vp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                bh, n, dk, dv, int(P))
    if rc:
        raise ValueError("%s rejected its arguments" % name)
    return out.reshape(tuple(lead) + (n, dv))


def recurrent_attention(q, k, v, P: int) -> np.ndarray:
    """O5: the fixed-size state form, S_p += phi_p(k) (x) [v, 1], read out as
    sum_p phi_p(q).S_p/(p! d^(p/2)) and normalised [hotdry, "Engineering
    realisation of the constant compute cost"].  fp64; tiny inputs only."""
    return _recurrent("orc_recurrent_attention", q, k, v, P)


def recurrent_attention_f32(q, k, v, P: int) -> np.ndarray:
    """O7: O5 with the state and arithmetic in float32 (diagnostic of the error
    that fp32 state accumulation carries by itself)."""
    return _recurrent("orc_recurrent_attention_f32", q, k, v, P)


def round_bf16(x) -> np.ndarray:
    """O8a: round to the nearest bfloat16 value, ties to even (8 significant
    bits, binary32 exponent range), returned as float64."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(a)
    _load().orc_round_bf16_array(a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                 out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), a.size)
    return out


def bf16_state_decode(q, k, v, P: int, n0: int, rounding: bool = True, window: int = 1) -> np.ndarray:
    """O8: decode steps on a bf16-stored state [hotdry, "Hardware optimisation
    paths and current limits": 16-bit storage of the state].  Tokens 0..n0-1
    are summed exactly into the one-sided state and rounded once; each later
    token is added exactly, read out from the unrounded sums and the sums are
    rounded to bf16 (ties to even) when stored.  Returns rows n0..n-1:
    [..., n - n0, d_V].  window > 1 stores only every window-th step: the
    steps between read out the stored values plus the exact terms of the
    tokens not yet stored.  rounding=False gives the exact one-sided recurrent
    form.  fp64; moderate inputs."""
    lead, bh, n, dk, dv = _heads(np.asarray(q), np.asarray(k), np.asarray(v))
    if not 0 <= n0 <= n:
        raise ValueError("need 0 <= n0 <= n")
    q32, qp = _f32(q)
    k32, kp = _f32(k)
    v32, vp = _f32(v)
    out = np.empty((bh, n - n0, dv), dtype=np.float64)
    rc = _load().orc_bf16_state_decode(qp, kp, vp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                       bh, int(n0), n, dk, dv, int(P), 1 if rounding else 0, int(window))
    if rc:
        raise ValueError("orc_bf16_state_decode rejected its arguments")
    return out.reshape(tuple(lead) + (n - n0, dv))


def round_f16(x) -> np.ndarray:
    """O8b: round to the nearest IEEE binary16 value, ties to even (11
    significant bits, gradual underflow below 2^-14, +-inf past 65504),
    returned as float64."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(a)
    _load().orc_round_f16_array(a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), a.size)
    return out


def f16_state_decode(q, k, v, P: int, n0: int, low_orders: int = 3, window: int = 1,
                     low_features: int | None = None) -> np.ndarray:
    """O8 for an fp16-stored state [hotdry, "Hardware optimisation paths and
    current limits": Float16 storage at P = 4]: as bf16_state_decode, but the
    first low_features features (numbered order by order; by default all those
    of the orders below low_orders) are stored in fp32 (round to nearest
    binary32) and the others in fp16 (round to nearest binary16, ties to
    even).  Returns rows n0..n-1: [..., n - n0, d_V].  fp64; moderate inputs."""
    lead, bh, n, dk, dv = _heads(np.asarray(q), np.asarray(k), np.asarray(v))
    if not 0 <= n0 <= n:
        raise ValueError("need 0 <= n0 <= n")
    if low_features is None:
        low_features = cumulative_basis(dk, low_orders) if low_orders > 0 else 0
    q32, qp = _f32(q)
    k32, kp = _f32(k)
    v32, vp = _f32(v)
    out = np.empty((bh, n - n0, dv), dtype=np.float64)
    rc = _load().orc_f16_state_decode(qp, kp, vp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                      bh, int(n0), n, dk, dv, int(P), int(low_features), int(window))
    if rc:
        raise ValueError("orc_f16_state_decode rejected its arguments")
    return out.reshape(tuple(lead) + (n - n0, dv))


def taylor_attention_grad(q, k, v, dout, P: int):
    """O9: dL/dq, dL/dk, dL/dv for L = sum(dout * O1(q, k, v)), by fp64 reverse-mode
    differentiation (torch autograd on CPU) of the quadratic definition
    x = q k^T / sqrt(d_K), w = sum_{p<P} x^p/p! on j <= i, o = (w v) / sum_j w
    [hotdry, "Core insight of symmetric tensor decomposition"].  One head at a
    time (n x n weights); inputs [..., n, d] as float32 values."""
    import torch
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    dout = np.asarray(dout, dtype=np.float32)
    lead, bh, n, dk, dv = _heads(q, k, v)
    outs = [np.empty((bh, n, dk)), np.empty((bh, n, dk)), np.empty((bh, n, dv))]
    qf, kf, vf, df = (a.reshape(bh, n, -1) for a in (q, k, v, dout))
    mask = torch.tril(torch.ones(n, n, dtype=torch.float64))
    for h in range(bh):
        Q = torch.tensor(qf[h], dtype=torch.float64, requires_grad=True)
        K = torch.tensor(kf[h], dtype=torch.float64, requires_grad=True)
        V = torch.tensor(vf[h], dtype=torch.float64, requires_grad=True)
        x = (Q @ K.T) / math.sqrt(dk)
        w = torch.zeros_like(x)
        term = torch.ones_like(x)
        for p in range(P):
            w = w + term
            term = term * x / (p + 1)
        W = w * mask
        o = (W @ V) / W.sum(dim=1, keepdim=True)
        o.backward(torch.tensor(df[h], dtype=torch.float64))
        for slot, t in enumerate((Q, K, V)):   # P = 1: o does not depend on q, k (no gradient)
            outs[slot][h] = t.grad.numpy() if t.grad is not None else 0.0
    return tuple(a.reshape(tuple(lead) + (n, -1)) for a in outs)


# ---------------------------------------------------------------- closed forms (O6)

def basis_size(d: int, p: int) -> int:
    """Minimal-basis size of one order: C(d+p-1, p)
    [hotdry, "Core insight of symmetric tensor decomposition"]."""
    return math.comb(d + p - 1, p)


def cumulative_basis(d: int, P: int) -> int:
    """Features over the orders 0..P-1: C(d+P-1, P-1), the factor in the state
    size [hotdry, "Engineering realisation of the constant compute cost"]."""
    return math.comb(d + P - 1, P - 1)


def state_size(d_k: int, d_v: int, P: int) -> int:
    """(d_V + 1) * C(d_K+P-1, P-1) values per head
    [hotdry, "Engineering realisation of the constant compute cost"]."""
    return (d_v + 1) * cumulative_basis(d_k, P)


def flops_per_token(d_k: int, d_v: int, P: int) -> Fraction:
    """(4 d_V + 2 (P d_K + 1)/(d_K + 1) + 2) * C(d_K+P-1, P-1), exactly
    [hotdry, "Engineering realisation of the constant compute cost"]."""
    return (4 * d_v + Fraction(2 * (P * d_k + 1), d_k + 1) + 2) * cumulative_basis(d_k, P)


def conventional_cost(n: int, d_k: int, d_v: int):
    """(KV-cache values, FLOPs) per token of softmax attention at context n
    [hotdry, "Scale bottleneck of conventional self-attention"]."""
    return n * (d_k + d_v), n * (2 * d_k + 2 * d_v + 3)
