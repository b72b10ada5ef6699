"""GPU parity of the deferred decode (decode window W > 1: W - 1 steps read
the state out and add the not-yet-stored tokens by their direct Taylor
weights, every W-th step folds them into the state) against the oracle.

fp32 state: against the quadratic definition (O1) at the fp32 bar, since the
outputs equal those of W = 1 up to rounding.  bf16 state: against O8 with the
same window (stores, and so roundings, only at the folds), at the bf16-state
bar of test_gpu_bf16_state.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import TOL_BF16, TOL_F32, decode, dev_all, prefill, rel_err, say

pytestmark = pytest.mark.gpu

TOL_BF16_STATE = 1e-3
DRIFT_SHARE = 1e-2


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as s
    s.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return s


def _steps(idx, st, q, k, v, lo, hi, out_dtype=torch.float32):
    outs = [decode(idx, st, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                   out_dtype=out_dtype) for t in range(lo, hi)]
    return torch.stack(outs, dim=2).float().cpu().numpy()


@pytest.mark.parametrize("window,n", [(2, 40), (5, 40), (16, 40), (64, 150)])
def test_window_from_empty_every_row_and_flushed_state(sata, oracle, window, n):
    d, P = 16, 4
    x = si.draw_qkv((2, 2), n, d, d, 3100 + window, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("decode window %d from empty, %d steps" % (window, n))
    st = sata.State(idx, 2, 2)
    sata.sata_state_set_decode_window(st, window)
    o = _steps(idx, st, q, k, v, 0, n)
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= TOL_F32
    # after a flush the buffer holds every token, as after plain steps
    sata.sata_state_flush(st)
    ref = sata.State(idx, 2, 2)
    _steps(idx, ref, q, k, v, 0, n)
    a, b = sata.state_tensor(st).cpu().numpy(), sata.state_tensor(ref).cpu().numpy()
    np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-5 * np.abs(b).max())


@pytest.mark.parametrize("d", [8, 32, 64])
@pytest.mark.parametrize("P", [1, 3, 4])
def test_window_all_shapes(sata, oracle, d, P):
    n, window = 11, 3
    x = si.draw_qkv((1, 3), n, d, d, 3200 + d + P, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("decode window %d d=%d P=%d" % (window, d, P))
    st = sata.State(idx, 1, 3)
    sata.sata_state_set_decode_window(st, window)
    o = _steps(idx, st, q, k, v, 0, n)
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= TOL_F32


def test_window_with_prefill_and_window_changes(sata, oracle):
    """prefill, 37 steps at W = 16 (two folds, five tokens pending), W = 1
    (folds them), 3 plain steps, W = 16 again, 4 deferred steps, a prefill
    continuation (folds them first), 18 more deferred steps: every output row
    against O1."""
    d, P = 64, 4
    n1, t1, t2, t3, n2, t4 = 300, 37, 3, 4, 70, 18
    n = n1 + t1 + t2 + t3 + n2 + t4
    x = si.draw_qkv((1, 2), n, d, d, 3300, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    sl = lambda a, lo, hi: a[:, :, lo:hi].contiguous()
    say("decode window with prefill and window changes, n=%d" % n)
    st = sata.State(idx, 1, 2)
    outs = [prefill(idx, st, sl(q, 0, n1), sl(k, 0, n1), sl(v, 0, n1)).cpu().numpy()]
    pos = n1
    sata.sata_state_set_decode_window(st, 16)
    outs.append(_steps(idx, st, q, k, v, pos, pos + t1)); pos += t1
    sata.sata_state_set_decode_window(st, 1)
    outs.append(_steps(idx, st, q, k, v, pos, pos + t2)); pos += t2
    sata.sata_state_set_decode_window(st, 16)
    outs.append(_steps(idx, st, q, k, v, pos, pos + t3)); pos += t3
    outs.append(prefill(idx, st, sl(q, pos, pos + n2), sl(k, pos, pos + n2), sl(v, pos, pos + n2)).cpu().numpy())
    pos += n2
    outs.append(_steps(idx, st, q, k, v, pos, pos + t4)); pos += t4
    o = np.concatenate(outs, axis=2)
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= TOL_F32


def test_window_bf16_io(sata, oracle):
    d, P, n, window = 32, 4, 30, 8
    x = si.draw_qkv((2, 2), n, d, d, 3400, "bf16")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("decode window %d, bf16 io" % window)
    st = sata.State(idx, 2, 2)
    sata.sata_state_set_decode_window(st, window)
    o = _steps(idx, st, q, k, v, 0, n, out_dtype=torch.bfloat16)
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= TOL_BF16


@pytest.mark.parametrize("d,n0,T,window", [(16, 256, 300, 16), (64, 128, 40, 16), (8, 64, 600, 4), (32, 100, 140, 64)])
def test_window_on_bf16_state_matches_emulation(sata, oracle, d, n0, T, window):
    P, heads = 4, 2
    x = si.draw_qkv((1, heads), n0 + T, d, d, 3500 + d, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("decode window %d on a bf16 state d=%d n0=%d T=%d" % (window, d, n0, T))
    st32 = sata.State(idx, 1, heads)
    prefill(idx, st32, q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous())
    st = sata.State(idx, 1, heads, dtype=torch.bfloat16)
    sata.sata_state_convert(st32, st)
    sata.sata_state_set_decode_window(st, window)
    o = _steps(idx, st, q, k, v, n0, n0 + T)
    ref = oracle.bf16_state_decode(x.q, x.k, x.v, P, n0, window=window)
    exact = oracle.taylor_attention(x.q, x.k, x.v, P, rows=np.arange(n0, n0 + T, dtype=np.int64))
    err, drift = rel_err(o, ref), rel_err(ref, exact)
    say("  err vs emulation %.3e, emulation drift %.3e" % (err, drift))
    assert err <= TOL_BF16_STATE + DRIFT_SHARE * drift


@pytest.mark.parametrize("window,steps", [(16, 20), (64, 70)])
def test_window_workload_d64_after_8192(sata, oracle, window, steps):
    """32 x 8 heads after an fp32 prefill of 8192 tokens, folds at every
    window-th step: every head of every step against O1."""
    wl = si.WORKLOADS["decode_d64_p4_f32"]
    say("decode window %d workload %s (%d steps)" % (window, wl.name, steps))
    pre = wl.draw()
    dec = wl.draw_decode(steps)
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    q, k, v = dev_all(pre)
    prefill(idx, st, q, k, v)
    del q, k, v
    sata.sata_state_set_decode_window(st, window)
    dq, dk_, dv_ = dev_all(dec)
    o = _steps(idx, st, dq, dk_, dv_, 0, steps)
    qa = np.concatenate([pre.q, dec.q], axis=2)
    ka = np.concatenate([pre.k, dec.k], axis=2)
    va = np.concatenate([pre.v, dec.v], axis=2)
    ref = oracle.taylor_attention(qa, ka, va, wl.P, rows=np.arange(wl.n, wl.n + steps, dtype=np.int64))
    err = rel_err(o, ref)
    say("  err %.3e" % err)
    assert err <= TOL_F32


def test_window_error_paths(sata):
    idx = sata.Index(16, 16, 4)
    st = sata.State(idx, 1, 1)
    for bad in (0, 65, -3):
        with pytest.raises(sata.SataError) as e:
            sata.sata_state_set_decode_window(st, bad)
        assert e.value.status == sata.SATA_ERR_INVALID
    sata.sata_state_flush(st)            # nothing pending: a no-op
