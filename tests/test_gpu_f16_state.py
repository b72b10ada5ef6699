"""GPU parity of the fp16-stored decode state (opt-in, decode only): binary16
words for the orders >= 2, fp32 for orders 0 and 1 (the first m_low features of
every row).  Compared with the oracle's emulation of it (O8, fp16 form: exact
sums, read out before the store, stored rounded -- to binary32 below m_low, to
binary16, ties to even, above) and with the exact Taylor attention (O1).

Bar against the emulation, on the usual metric (max over rows of the normwise
relative error): TOL_F16_STATE + DRIFT_SHARE * drift, drift being the
emulation's own distance from the exact result.  Where the kernel's fp32 sum
and the oracle's fp64 sum fall on either side of a binary16 half-way point the
two store neighbouring values, one fp16 ulp (2^-11 relative) apart, and the
runs carry different rounding errors from then on; both that difference and
the drift grow with the readout's conditioning.  A kernel that stored the low
orders in fp16, truncated, or read out after rounding would sit about one
drift (or, for the low orders, far more) away.  Against O1 the bar is the bf16
paths' 2e-2, over all 1024 steps of the decode workload.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import TOL_BF16, decode, dev_all, prefill, rel_err, say

pytestmark = pytest.mark.gpu

TOL_F16_STATE = 2e-4
DRIFT_SHARE = 1e-2
def _m_low(sata, st):
    """The state's fp32 features (orders 0 and 1, rounded up to 64)."""
    return sata.state_low_tensor(st).shape[-1]


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as s
    s.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return s


def _f16_state_from_prefill(sata, idx, B, H, q, k, v):
    """fp32 prefill of the given tokens, then conversion into a new fp16 state."""
    st32 = sata.State(idx, B, H)
    if q.shape[2]:
        prefill(idx, st32, q, k, v)
    st16 = sata.State(idx, B, H, dtype=torch.float16)
    sata.sata_state_convert(st32, st16)
    return st32, st16


def _steps(idx, st, q, k, v, lo, hi):
    outs = [decode(idx, st, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous())
            for t in range(lo, hi)]
    return torch.stack(outs, dim=2).cpu().numpy()


@pytest.mark.parametrize("d,P", [(16, 4), (64, 3), (8, 1)])
def test_f16_convert_keeps_low_orders_in_fp32(sata, d, P):
    """fp32 -> fp16: features below m_low copied exactly into the fp32 part (their
    fp16 slots zero), the rest rounded to nearest even; fp16 -> fp32 gives
    back exactly those values."""
    n = 300
    x = si.draw_qkv((2, 3), n, d, d, 4343 + d, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("fp16 state convert d=%d P=%d" % (d, P))
    st32, st16 = _f16_state_from_prefill(sata, idx, 2, 3, q, k, v)
    s32 = sata.state_tensor(st32).clone()
    main = sata.state_tensor(st16).clone()
    low = sata.state_low_tensor(st16).clone()
    m_low = low.shape[-1]
    assert m_low == min(-(-(1 + d) // 64) * 64, idx.m_pad)
    assert torch.equal(low, s32[..., :m_low])
    assert torch.all(main[..., :m_low] == 0)
    assert torch.equal(main[..., m_low:].view(torch.int16), s32[..., m_low:].to(torch.float16).view(torch.int16))
    back = sata.State(idx, 2, 3)
    sata.sata_state_convert(st16, back)
    wide = sata.state_tensor(back)
    assert torch.equal(wide[..., :m_low], s32[..., :m_low])
    assert torch.equal(wide[..., m_low:], main[..., m_low:].float())
    for s in (st32, st16, back):
        s.free()
    idx.free()


@pytest.mark.parametrize("d,P,n0,T,heads", [
    (16, 4, 300, 24, 2),
    (64, 4, 200, 12, 2),
    (32, 3, 0, 20, 2),      # from an empty state
    (8, 2, 77, 30, 3),
    (64, 1, 50, 10, 2),     # one feature: all of it in the fp32 part
])
def test_f16_state_decode_matches_emulation(sata, oracle, d, P, n0, T, heads):
    x = si.draw_qkv((1, heads), n0 + T, d, d, 950 + d + n0, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("fp16-state decode d=%d P=%d n0=%d T=%d heads=%d" % (d, P, n0, T, heads))
    _, st = _f16_state_from_prefill(sata, idx, 1, heads, q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(),
                                    v[:, :, :n0].contiguous())
    o = _steps(idx, st, q, k, v, n0, n0 + T)
    ref = oracle.f16_state_decode(x.q, x.k, x.v, P, n0, low_features=_m_low(sata, st))
    exact = oracle.taylor_attention(x.q, x.k, x.v, P)[:, :, n0:]
    err, drift, err_exact = rel_err(o, ref), rel_err(ref, exact), rel_err(o, exact)
    say("  err vs emulation %.3e, drift %.3e, err vs exact %.3e" % (err, drift, err_exact))
    assert err <= TOL_F16_STATE + DRIFT_SHARE * drift
    assert err_exact <= TOL_BF16


@pytest.mark.parametrize("window", [1, 4])
def test_f16_state_whole_tile_grid(sata, oracle, window):
    """43 x 8 heads at d = 64 (24 tiles of 2048 fp16 features each: 8256 tile
    workgroups, past the row-split threshold) so the whole-tile step and read
    kernels run; window 4 adds the fold and three read steps per fold.  Two
    sampled heads against the emulation."""
    d, P, B, H, n0, T = 64, 4, 43, 8, 64, 8
    x = si.draw_qkv((B, H), n0 + T, d, d, 977 + window, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("fp16-state decode whole-tile grid, %d x %d heads, window %d" % (B, H, window))
    st32, st = _f16_state_from_prefill(sata, idx, B, H, q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(),
                                       v[:, :, :n0].contiguous())
    st32.free()
    if window > 1:
        sata.sata_state_set_decode_window(st, window)
    o = _steps(idx, st, q, k, v, n0, n0 + T)
    for b, h in ((0, 0), (B - 1, H - 1)):
        sub = lambda a: np.ascontiguousarray(a[b:b + 1, h:h + 1])
        ref = oracle.f16_state_decode(sub(x.q), sub(x.k), sub(x.v), P, n0, window=window,
                                      low_features=_m_low(sata, st))
        exact = oracle.taylor_attention(sub(x.q), sub(x.k), sub(x.v), P)[:, :, n0:]
        err, drift = rel_err(o[b:b + 1, h:h + 1], ref), rel_err(ref, exact)
        say("  head (%d, %d): err vs emulation %.3e, drift %.3e" % (b, h, err, drift))
        assert err <= TOL_F16_STATE + DRIFT_SHARE * drift
    st.free()
    idx.free()


def test_f16_state_window_and_flush(sata, oracle):
    """Window 4 over 12 steps (three folds) against the emulation with the same
    window; then 2 more steps left pending, a flush, and a plain step against the
    same steps run plainly on a second fp16 state (one rounding apart)."""
    d, P, n0, heads = 32, 4, 100, 2
    x = si.draw_qkv((1, heads), n0 + 15, d, d, 991, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("fp16-state decode window 4 and flush, d=%d" % d)
    pre = lambda a: a[:, :, :n0].contiguous()
    _, st = _f16_state_from_prefill(sata, idx, 1, heads, pre(q), pre(k), pre(v))
    _, plain = _f16_state_from_prefill(sata, idx, 1, heads, pre(q), pre(k), pre(v))
    sata.sata_state_set_decode_window(st, 4)
    o = _steps(idx, st, q, k, v, n0, n0 + 12)
    ref = oracle.f16_state_decode(x.q[:, :, :n0 + 12], x.k[:, :, :n0 + 12], x.v[:, :, :n0 + 12], P, n0,
                                  window=4, low_features=_m_low(sata, st))
    exact = oracle.taylor_attention(x.q, x.k, x.v, P)
    err, drift = rel_err(o, ref), rel_err(ref, exact[:, :, n0:n0 + 12])
    say("  window: err vs emulation %.3e, drift %.3e" % (err, drift))
    assert err <= TOL_F16_STATE + DRIFT_SHARE * drift
    _steps(idx, st, q, k, v, n0 + 12, n0 + 14)
    sata.sata_state_flush(st)
    sata.sata_state_set_decode_window(st, 1)
    last = _steps(idx, st, q, k, v, n0 + 14, n0 + 15)
    _steps(idx, plain, q, k, v, n0, n0 + 14)
    last_plain = _steps(idx, plain, q, k, v, n0 + 14, n0 + 15)
    e1, e2 = rel_err(last, exact[:, :, n0 + 14:]), rel_err(last, last_plain)
    say("  after flush: err vs exact %.3e, vs plain steps %.3e" % (e1, e2))
    assert e1 <= TOL_BF16 and e2 <= 1e-3
    st.free()
    plain.free()
    idx.free()


def test_f16_state_d128(sata, oracle):
    """Head size 128 (the row-split kernels, nine column tiles; m_low = 136)."""
    d, P, n0, T, heads = 128, 3, 70, 4, 2
    x = si.draw_qkv((1, heads), n0 + T, d, d, 9500, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("fp16-state decode d=128 P=%d n0=%d" % (P, n0))
    _, st = _f16_state_from_prefill(sata, idx, 1, heads, q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(),
                                    v[:, :, :n0].contiguous())
    o = _steps(idx, st, q, k, v, n0, n0 + T)
    ref = oracle.f16_state_decode(x.q, x.k, x.v, P, n0, low_features=_m_low(sata, st))
    exact = oracle.taylor_attention(x.q, x.k, x.v, P)[:, :, n0:]
    err, drift = rel_err(o, ref), rel_err(ref, exact)
    say("  err vs emulation %.3e, drift %.3e" % (err, drift))
    assert err <= TOL_F16_STATE + DRIFT_SHARE * drift
    st.free()
    idx.free()


@pytest.mark.parametrize("wl_name,pairs", [("decode_d64_p4_f32", ((0, 0), (31, 7)))])
def test_f16_state_1024_steps_against_exact(sata, oracle, wl_name, pairs):
    """The decode workload (32 x 8 heads, d = 64, P = 4): fp32 prefill of 8192
    tokens converted to fp16, then all 1024 decode steps; every step of two
    sampled heads against the exact Taylor attention (O1) at 2e-2."""
    wl = si.WORKLOADS[wl_name]
    steps = wl.decode_steps
    pre = wl.draw()
    dec = si.draw_qkv((wl.batch, wl.heads), steps, wl.d_k, wl.d_v, wl.seed + 31, "f32")
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    q, k, v = dev_all(pre)
    say("fp16-state decode %s: %d steps after %d tokens" % (wl.name, steps, wl.n))
    st32, st = _f16_state_from_prefill(sata, idx, wl.batch, wl.heads, q, k, v)
    st32.free()
    del q, k, v
    qd, kd, vd = dev_all(dec)
    o = _steps(idx, st, qd, kd, vd, 0, steps)
    worst = 0.0
    for b, h in pairs:
        cat = lambda a, c: np.concatenate([a[b:b + 1, h:h + 1], c[b:b + 1, h:h + 1]], axis=2)
        rows = np.arange(wl.n, wl.n + steps)
        ref = oracle.taylor_attention(cat(pre.q, dec.q), cat(pre.k, dec.k), cat(pre.v, dec.v), wl.P, rows=rows)
        err = rel_err(o[b:b + 1, h:h + 1], ref)
        say("  head (%d, %d): err vs exact over %d steps %.3e" % (b, h, steps, err))
        worst = max(worst, err)
    assert worst <= TOL_BF16
    st.free()
    idx.free()


def test_f16_state_refused_for_prefill(sata):
    idx = sata.Index(16, 16, 3)
    st = sata.State(idx, 1, 1, dtype=torch.float16)
    x = torch.zeros((1, 1, 8, 16), device="cuda")
    with pytest.raises(sata.SataError) as e:
        prefill(idx, st, x, x, x)
    assert e.value.status == sata.SATA_ERR_UNSUPPORTED
    st.free()
    idx.free()
