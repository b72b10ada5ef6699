"""ctypes binding of libsata.so (argument marshalling only).

The functions keep the C names of include/sata.h.  Tensors are torch tensors
on the GPU (torch provides device memory and streams; every step of the
computation runs in the library's HIP kernels).  There is no CPU fallback:
if libsata.so is missing or fails to load, every call raises.

Citations are those of include/sata.h ([hotdry] blog.hotdry.top,
"Symmetry-aware Taylor approximation attention: engineering a constant
per-token cost", 2026-02-05).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsata.so")

SATA_OK, SATA_ERR_INVALID, SATA_ERR_UNSUPPORTED, SATA_ERR_OOM, SATA_ERR_HIP = range(5)
SATA_NOALLOC_SCRATCH_BYTES = 128 << 20   # include/sata.h
SATA_F32, SATA_BF16, SATA_F16 = 0, 1, 2

_EXPORTS = (
    "sata_build_index", "sata_index_free", "sata_index_features", "sata_index_info",
    "sata_state_alloc", "sata_state_alloc_dtype", "sata_state_convert", "sata_state_set_decode_window",
    "sata_state_flush", "sata_state_check", "sata_state_reset", "sata_state_free",
    "sata_state_data",
    "sata_prefill", "sata_prefill_noalloc", "sata_prefill_backward", "sata_decode_step", "sata_expand_features", "sata_describe_features", "sata_describe_quads",
    "sata_describe_quads16",
    "sata_status_string", "sata_last_error",
    "sata_profile_enable", "sata_profile_query", "sata_profile_kernel_name",
    "sata_describe_prefill_plan", "sata_debug_scan_faults", "sata_debug_prefill_positions", "sata_debug_prefill_refresh",
    "sata_measure_mfma_loop",
)

_lib = None


class SataError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (func, _STATUS.get(status, "status %d" % status), detail))


_STATUS = {
    SATA_ERR_INVALID: "SATA_ERR_INVALID",
    SATA_ERR_UNSUPPORTED: "SATA_ERR_UNSUPPORTED",
    SATA_ERR_OOM: "SATA_ERR_OOM",
    SATA_ERR_HIP: "SATA_ERR_HIP",
}


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libsata.so (built in-tree by constant_cost_attention_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libsata.so not found at %s: build it with "
                           "`python -m constant_cost_attention_amd.build`" % p)
    lib = ctypes.CDLL(p)
    vp, i64, cint = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    pvp = ctypes.POINTER(ctypes.c_void_p)
    lib.sata_build_index.argtypes = [cint, cint, cint, pvp]
    lib.sata_index_free.argtypes = [vp]
    lib.sata_index_free.restype = None
    lib.sata_index_features.argtypes = [vp]
    lib.sata_index_features.restype = i64
    lib.sata_index_info.argtypes = [vp, ctypes.POINTER(cint), ctypes.POINTER(cint), ctypes.POINTER(cint),
                                    ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.sata_state_alloc.argtypes = [vp, cint, cint, vp, pvp]
    lib.sata_state_alloc_dtype.argtypes = [vp, cint, cint, cint, vp, pvp]
    lib.sata_state_convert.argtypes = [vp, vp, vp]
    lib.sata_state_set_decode_window.argtypes = [vp, cint, vp]
    lib.sata_state_flush.argtypes = [vp, vp]
    lib.sata_state_check.argtypes = [vp, vp]
    lib.sata_debug_scan_faults.argtypes = [cint, cint]
    lib.sata_debug_prefill_positions.argtypes = [cint]
    lib.sata_debug_prefill_refresh.argtypes = [cint]
    lib.sata_describe_prefill_plan.argtypes = [cint, cint, i64, i64, cint, cint, i64, ctypes.POINTER(i64),
                                               ctypes.POINTER(i64)]
    lib.sata_describe_prefill_plan.restype = i64
    lib.sata_state_reset.argtypes = [vp, vp]
    lib.sata_state_free.argtypes = [vp]
    lib.sata_state_free.restype = None
    lib.sata_state_data.argtypes = [vp, pvp, ctypes.POINTER(i64)]
    lib.sata_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i64, cint, cint, cint, vp]
    lib.sata_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, cint, cint, cint, vp]
    lib.sata_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, cint, cint, vp]
    lib.sata_prefill_backward.argtypes = [vp, cint, cint, vp, vp, vp, vp, vp, vp, vp, i64, cint, cint, cint, vp]
    lib.sata_expand_features.argtypes = [vp, vp, vp, i64, cint, cint, vp]
    lib.sata_describe_features.argtypes = [cint, cint, ctypes.POINTER(ctypes.c_uint32),
                                           ctypes.POINTER(ctypes.c_float), i64]
    lib.sata_describe_features.restype = i64
    lib.sata_describe_quads.argtypes = [cint, cint, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_float), i64]
    lib.sata_describe_quads.restype = i64
    lib.sata_describe_quads16.argtypes = [cint, cint, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_uint32), i64]
    lib.sata_describe_quads16.restype = i64
    lib.sata_status_string.argtypes = [cint]
    lib.sata_status_string.restype = ctypes.c_char_p
    lib.sata_last_error.argtypes = []
    lib.sata_last_error.restype = ctypes.c_char_p
    lib.sata_measure_mfma_loop.argtypes = [cint, ctypes.POINTER(ctypes.c_double)]
    lib.sata_measure_mfma_loop.restype = cint
    lib.sata_profile_enable.argtypes = [cint]
    lib.sata_profile_query.argtypes = [cint, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.sata_profile_kernel_name.argtypes = [cint]
    lib.sata_profile_kernel_name.restype = ctypes.c_char_p
    for name in ("sata_profile_enable", "sata_profile_query", "sata_build_index", "sata_index_info", "sata_state_alloc", "sata_state_alloc_dtype",
                 "sata_state_convert", "sata_state_set_decode_window", "sata_state_flush", "sata_state_check",
                 "sata_debug_scan_faults", "sata_debug_prefill_positions", "sata_debug_prefill_refresh",
                 "sata_state_reset",
                 "sata_state_data", "sata_prefill", "sata_prefill_noalloc", "sata_prefill_backward", "sata_decode_step",
                 "sata_expand_features"):
        getattr(lib, name).restype = cint
    _lib = lib
    return lib


def _check(status: int, func: str):
    if status != SATA_OK:
        raise SataError(status, func, load().sata_last_error().decode())


_DTYPES = {torch.float32: SATA_F32, torch.bfloat16: SATA_BF16}
_STATE_DTYPES = {torch.float32: SATA_F32, torch.bfloat16: SATA_BF16, torch.float16: SATA_F16}


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SATA_F32
    if t.dtype == torch.bfloat16:
        return SATA_BF16
    raise TypeError("dtype %s not supported (float32 or bfloat16)" % t.dtype)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev_ptr(t: torch.Tensor, name: str) -> ctypes.c_void_p:
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


class Index:
    """Handle of sata_index (M_p tables for one (d_K, d_V, P))."""

    def __init__(self, d_k: int, d_v: int, P: int):
        self.ptr = sata_build_index(d_k, d_v, P)
        self.d_k, self.d_v, self.P = d_k, d_v, P
        info = sata_index_info(self)
        self.m, self.m_pad = info["m"], info["m_pad"]

    def free(self):
        if self.ptr:
            sata_index_free(self)
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class State:
    """Handle of sata_state (fixed-size state of batch x heads heads); dtype is
    torch.float32 (default), torch.float16 or torch.bfloat16 (the last two
    decode only; float16 keeps orders 0 and 1 in float32)."""

    def __init__(self, index: Index, batch: int, heads: int, stream=None, dtype=torch.float32):
        self.index = index
        self.batch, self.heads = batch, heads
        self.dtype = dtype
        if dtype == torch.float32:
            self.ptr = sata_state_alloc(index, batch, heads, stream)
        else:
            self.ptr = sata_state_alloc_dtype(index, batch, heads, _STATE_DTYPES.get(dtype, -1), stream)

    def free(self):
        if self.ptr:
            sata_state_free(self)
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


# ---------------------------------------------------------------- C-named calls

def sata_build_index(d_k: int, d_v: int, P: int) -> ctypes.c_void_p:
    out = ctypes.c_void_p()
    _check(load().sata_build_index(int(d_k), int(d_v), int(P), ctypes.byref(out)), "sata_build_index")
    return out


def sata_index_free(index: Index):
    load().sata_index_free(index.ptr)


def sata_index_features(index: Index) -> int:
    return int(load().sata_index_features(index.ptr))


def sata_index_info(index: Index) -> dict:
    dk, dv, P = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    m, mp = ctypes.c_int64(), ctypes.c_int64()
    _check(load().sata_index_info(index.ptr, ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(P),
                                  ctypes.byref(m), ctypes.byref(mp)), "sata_index_info")
    return {"d_k": dk.value, "d_v": dv.value, "P": P.value, "m": m.value, "m_pad": mp.value}


def sata_state_alloc(index: Index, batch: int, heads: int, stream=None) -> ctypes.c_void_p:
    out = ctypes.c_void_p()
    _check(load().sata_state_alloc(index.ptr, int(batch), int(heads), _stream(stream), ctypes.byref(out)),
           "sata_state_alloc")
    return out


def sata_state_alloc_dtype(index: Index, batch: int, heads: int, state_dt: int, stream=None) -> ctypes.c_void_p:
    out = ctypes.c_void_p()
    _check(load().sata_state_alloc_dtype(index.ptr, int(batch), int(heads), int(state_dt), _stream(stream),
                                         ctypes.byref(out)), "sata_state_alloc_dtype")
    return out


def sata_state_convert(src: State, dst: State, stream=None):
    """Copy src into dst, converting the element type (fp32 -> bf16 rounds to nearest even)."""
    _check(load().sata_state_convert(src.ptr, dst.ptr, _stream(stream)), "sata_state_convert")


def sata_state_set_decode_window(state: State, window: int, stream=None):
    """Decode steps per state update (1..64); deferred tokens are read out from their direct weights."""
    _check(load().sata_state_set_decode_window(state.ptr, int(window), _stream(stream)),
           "sata_state_set_decode_window")


def sata_state_flush(state: State, stream=None):
    """Fold deferred decode tokens into the state buffer."""
    _check(load().sata_state_flush(state.ptr, _stream(stream)), "sata_state_flush")


def sata_state_check(state: State, stream=None):
    """Synchronise the stream; raise SataError(SATA_ERR_HIP) if asynchronous work on the state
    recorded a failure (a prefill scan item that gave up waiting for its predecessor)."""
    _check(load().sata_state_check(state.ptr, _stream(stream)), "sata_state_check")


def sata_debug_scan_faults(item_base: int = 0, spin_limit: int = 0):
    """Fault injection for tests of the scan's error path; (0, 0) restores the defaults."""
    _check(load().sata_debug_scan_faults(int(item_base), int(spin_limit)), "sata_debug_scan_faults")


def sata_debug_prefill_positions(mt: int = 0):
    """Force the fp16-operand scan's positions per update wavefront (measurement only; 0 = the rule)."""
    _check(load().sata_debug_prefill_positions(int(mt)), "sata_debug_prefill_positions")


def sata_debug_prefill_refresh(chunks: int = 0):
    """Force the fp16-operand scan's chunks per state-copy refresh (measurement only; 0 = the rule)."""
    _check(load().sata_debug_prefill_refresh(int(chunks)), "sata_debug_prefill_refresh")


def sata_describe_prefill_plan(d_k: int, P: int, batch_heads: int, n: int, chunk: int = 0, in_dt: int = SATA_BF16,
                               work_cap: int = 16 << 30) -> dict:
    """Host-only: workspace bytes, chunks per segment and slices per head of the chunked prefill."""
    lib = load()
    seg, sl = ctypes.c_int64(), ctypes.c_int64()
    wb = lib.sata_describe_prefill_plan(int(d_k), int(P), int(batch_heads), int(n), int(chunk), int(in_dt),
                                        int(work_cap), ctypes.byref(seg), ctypes.byref(sl))
    if wb < 0:
        raise SataError(SATA_ERR_INVALID, "sata_describe_prefill_plan", lib.sata_last_error().decode())
    return {"work_bytes": wb, "seg_chunks": seg.value, "slices": sl.value}


def sata_measure_mfma_loop(bf16: bool = True) -> float:
    """Dense TFLOP/s of a plain 16x16x32 MFMA loop on the current device (a measured ceiling)."""
    t = ctypes.c_double()
    _check(load().sata_measure_mfma_loop(1 if bf16 else 0, ctypes.byref(t)), "sata_measure_mfma_loop")
    return t.value


def sata_state_reset(state: State, stream=None):
    _check(load().sata_state_reset(state.ptr, _stream(stream)), "sata_state_reset")


def sata_state_free(state: State):
    load().sata_state_free(state.ptr)


def sata_state_data(state: State):
    """(device pointer, bytes) of the state buffer."""
    p, n = ctypes.c_void_p(), ctypes.c_int64()
    _check(load().sata_state_data(state.ptr, ctypes.byref(p), ctypes.byref(n)), "sata_state_data")
    return p.value, n.value


class _CudaArray:
    """Minimal __cuda_array_interface__ exporter so torch can view library memory."""

    def __init__(self, ptr: int, shape, typestr: str):
        self.__cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr,
                                         "data": (ptr, False), "version": 2, "strides": None}


def state_tensor(state: State) -> torch.Tensor:
    """The state buffer viewed as a tensor [B, H, d_V+1, m_pad] of the state's dtype (no copy)."""
    ptr, nbytes = sata_state_data(state)
    idx = state.index
    shape = (state.batch, state.heads, idx.d_v + 1, idx.m_pad)
    if state.dtype == torch.float32:
        assert nbytes == 4 * shape[0] * shape[1] * shape[2] * shape[3]
        return torch.as_tensor(_CudaArray(ptr, shape, "<f4"), device="cuda")
    if state.dtype == torch.float16:   # the binary16 array; the fp32 orders: state_low_tensor
        assert nbytes >= 2 * shape[0] * shape[1] * shape[2] * shape[3]
        return torch.as_tensor(_CudaArray(ptr, shape, "<f2"), device="cuda")
    assert nbytes == 2 * shape[0] * shape[1] * shape[2] * shape[3]
    return torch.as_tensor(_CudaArray(ptr, shape, "<i2"), device="cuda").view(torch.bfloat16)


def state_low_tensor(state: State) -> torch.Tensor:
    """An fp16 state's fp32 words of orders 0 and 1: [B, H, d_V+1, m_low] (no copy)."""
    if state.dtype != torch.float16:
        raise ValueError("only float16 states keep an fp32 part")
    ptr, nbytes = sata_state_data(state)
    idx = state.index
    rows = state.batch * state.heads * (idx.d_v + 1)
    main = 2 * rows * idx.m_pad
    m_low = (nbytes - main) // (4 * rows)
    return torch.as_tensor(_CudaArray(ptr + main, (state.batch, state.heads, idx.d_v + 1, m_low), "<f4"),
                           device="cuda")


def _prefill_args(index: Index, state: State, q, k, v, out):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, n, d_K]")
    B, H, n, dk = q.shape
    if (B, H) != (state.batch, state.heads) or dk != index.d_k:
        raise ValueError("q shape %s does not match the state (%d, %d, n, %d)" % (tuple(q.shape), state.batch,
                                                                                  state.heads, index.d_k))
    if k.shape != q.shape or v.shape != (B, H, n, index.d_v) or out.shape != v.shape:
        raise ValueError("k, v, out shapes disagree with q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    return n


def sata_prefill(index: Index, state: State, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 out: torch.Tensor, chunk: int = 0, stream=None):
    """q, k: [B, H, n, d_K]; v, out: [B, H, n, d_V] on the GPU."""
    n = _prefill_args(index, state, q, k, v, out)
    _check(load().sata_prefill(index.ptr, state.ptr, _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                               _dev_ptr(out, "out"), int(n), int(chunk), _dtype(q), _dtype(out),
                               _stream(stream)), "sata_prefill")
    return out


def sata_prefill_noalloc(index: Index, state: State, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         out: torch.Tensor, chunk: int = 0, stream=None):
    """sata_prefill without device allocation (workspace: the library's per-device scratch array)."""
    n = _prefill_args(index, state, q, k, v, out)
    _check(load().sata_prefill_noalloc(index.ptr, state.ptr, _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                       _dev_ptr(out, "out"), int(n), int(chunk), _dtype(q), _dtype(out),
                                       _stream(stream)), "sata_prefill_noalloc")
    return out


def sata_prefill_backward(index: Index, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
                          dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, chunk: int = 0, stream=None):
    """Gradients of a causal prefill from a zero state: q, k, v, dout, dq, dk, dv all [B, H, n, d]."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, n, d_K]")
    B, H, n, dk_ = q.shape
    if dk_ != index.d_k or index.d_k != index.d_v:
        raise ValueError("q's last dim must be d_K (== d_V)")
    for name, t in (("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape:
            raise ValueError("%s must have q's shape %s" % (name, tuple(q.shape)))
    if k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype:
        raise ValueError("q, k, v, dout must share a dtype")
    if dk.dtype != dq.dtype or dv.dtype != dq.dtype:
        raise ValueError("dq, dk, dv must share a dtype")
    _check(load().sata_prefill_backward(index.ptr, int(B), int(H), _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                        _dev_ptr(dout, "dout"), _dev_ptr(dq, "dq"), _dev_ptr(dk, "dk"),
                                        _dev_ptr(dv, "dv"), int(n), int(chunk), _dtype(q), _dtype(dq),
                                        _stream(stream)), "sata_prefill_backward")
    return dq, dk, dv


def sata_decode_step(index: Index, state: State, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     out: torch.Tensor, stream=None):
    """q, k: [B, H, d_K] (or [B, H, 1, d_K]); v, out: [B, H, d_V] (or [B, H, 1, d_V])."""
    B, H = state.batch, state.heads
    if q.numel() != B * H * index.d_k or k.shape != q.shape:
        raise ValueError("q, k must hold [B, H, d_K] values")
    if v.numel() != B * H * index.d_v or out.numel() != v.numel():
        raise ValueError("v, out must hold [B, H, d_V] values")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    _check(load().sata_decode_step(index.ptr, state.ptr, _dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                   _dev_ptr(out, "out"), _dtype(q), _dtype(out), _stream(stream)),
           "sata_decode_step")
    return out


def sata_expand_features(index: Index, x: torch.Tensor, out: torch.Tensor, side: int, stream=None):
    """x: [rows, d_K]; out: [rows, m_pad] float32; side 0 = key monomials, 1 = query-side weights."""
    rows = x.shape[0] if x.dim() > 1 else 1
    if x.numel() != rows * index.d_k or out.numel() != rows * index.m_pad or out.dtype != torch.float32:
        raise ValueError("x must be [rows, d_K], out [rows, m_pad] float32")
    _check(load().sata_expand_features(index.ptr, _dev_ptr(x, "x"), _dev_ptr(out, "out"), int(rows), int(side),
                                       _dtype(x), _stream(stream)), "sata_expand_features")
    return out


def sata_describe_features(d_k: int, P: int):
    """Host-only: (tuples uint32 [m], coef float32 [m]) of the tables sata_build_index uploads."""
    import numpy as np
    lib = load()
    m = lib.sata_describe_features(int(d_k), int(P), None, None, 0)
    if m < 0:
        raise SataError(SATA_ERR_UNSUPPORTED if d_k > 0 and P >= 1 else SATA_ERR_INVALID, "sata_describe_features",
                        lib.sata_last_error().decode())
    tup = np.zeros(m, dtype=np.uint32)
    coef = np.zeros(m, dtype=np.float32)
    lib.sata_describe_features(int(d_k), int(P), tup.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                               coef.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), m)
    return tup, coef


PROFILE_KERNELS = {"prefill_scan": 0, "prefill_combine": 1, "decode_stream": 2, "decode_finish": 3,
                   "decode_read": 4, "decode_fold": 5, "decode_low": 6}


def sata_profile_enable(on: bool):
    _check(load().sata_profile_enable(1 if on else 0), "sata_profile_enable")


def sata_profile_query(kernel) -> tuple:
    """(summed milliseconds, launches) of one kernel's recorded event pairs."""
    kid = PROFILE_KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(load().sata_profile_query(kid, ctypes.byref(ms), ctypes.byref(n)), "sata_profile_query")
    return ms.value, n.value


def sata_profile_kernel_name(kernel: int):
    r = load().sata_profile_kernel_name(int(kernel))
    return r.decode() if r else None


def sata_describe_quads(d_k: int, P: int):
    """Host-only: (w0 uint32 [nq], cidx int32 [nq], coef float32 [nq, 4]) of the prefill's quads."""
    import numpy as np
    lib = load()
    nq = lib.sata_describe_quads(int(d_k), int(P), None, None, None, 0)
    if nq < 0:
        raise SataError(SATA_ERR_UNSUPPORTED if d_k > 0 and P >= 1 else SATA_ERR_INVALID, "sata_describe_quads",
                        lib.sata_last_error().decode())
    w0 = np.zeros(nq, dtype=np.uint32)
    cidx = np.zeros(nq, dtype=np.int32)
    coef = np.zeros((nq, 4), dtype=np.float32)
    lib.sata_describe_quads(int(d_k), int(P), w0.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                            cidx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            coef.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), nq)
    return w0, cidx, coef


def sata_describe_quads16(d_k: int, P: int):
    """Host-only: (w0 uint32 [np, 16], cidx int32 [np, 16], coef float32 [np, 16, 4],
    flags uint32 [np]) of the fp16-operand scan's positions (np = 0 outside its range)."""
    import numpy as np
    lib = load()
    npos = lib.sata_describe_quads16(int(d_k), int(P), None, None, None, None, 0)
    if npos < 0:
        raise SataError(SATA_ERR_UNSUPPORTED if d_k > 0 and P >= 1 else SATA_ERR_INVALID, "sata_describe_quads16",
                        lib.sata_last_error().decode())
    w0 = np.zeros((npos, 16), dtype=np.uint32)
    cidx = np.zeros((npos, 16), dtype=np.int32)
    coef = np.zeros((npos, 16, 4), dtype=np.float32)
    flags = np.zeros(npos, dtype=np.uint32)
    lib.sata_describe_quads16(int(d_k), int(P), w0.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                              cidx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                              coef.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                              flags.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), npos)
    return w0, cidx, coef, flags


def status_string(status: int) -> str:
    return load().sata_status_string(int(status)).decode()


def exported_symbols() -> tuple:
    return _EXPORTS
