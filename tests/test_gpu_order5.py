"""Five orders (P = 5: features up to degree 4, each a three-index prefix
times an aligned block of last indices in the prefill's quad view) through
every entry point: expansion, prefill (fp32 and bf16 inputs), decode (plain,
windowed, bf16-stored state), backward, against the oracle (O1, O8, O9)."""
import math

import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import TOL_BF16, TOL_F32, decode, dev_all, prefill, rel_err, sample_rows, say

pytestmark = pytest.mark.gpu

P = 5


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as s
    s.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return s


def _tol(dtype):
    return TOL_F32 if dtype == "f32" else TOL_BF16


@pytest.mark.parametrize("d", [8, 16, 32])
def test_expand_order5_matches_bruteforce_basis(sata, oracle, d):
    say("expand d=%d P=5" % d)
    idx = sata.Index(d, d, P)
    x = si.draw_qkv((1,), 5, d, d, 7770 + d, "f32").q[0]
    xt = torch.from_numpy(x).cuda()
    outs = []
    for side in (0, 1):
        o = torch.zeros((5, idx.m_pad), dtype=torch.float32, device="cuda")
        sata.sata_expand_features(idx, xt, o, side)
        outs.append(o.cpu().numpy().astype(np.float64))
    xd = x.astype(np.float64)
    f = 0
    for p in range(P):
        tup, cnt = oracle.basis_bruteforce(d, p)
        mono = np.prod(xd[:, tup], axis=-1) if p else np.ones((5, 1))
        w = cnt / (math.factorial(p) * math.sqrt(d) ** p)
        g = len(cnt)
        np.testing.assert_allclose(outs[0][:, f:f + g], mono, rtol=6e-7, atol=1e-30)
        np.testing.assert_allclose(outs[1][:, f:f + g], mono * w, rtol=1e-6, atol=1e-30)
        f += g
    assert f == idx.m and np.all(outs[0][:, f:] == 0) and np.all(outs[1][:, f:] == 0)
    idx.free()


@pytest.mark.parametrize("d", [8, 16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_order5_every_row(sata, oracle, d, dtype):
    chunk = 128 if d == 64 else 64
    n = 2 * chunk + 37
    heads = 2 if d == 64 else 3
    say("prefill P=5 d=%d %s n=%d" % (d, dtype, n))
    x = si.draw_qkv((1, heads), n, d, d, 5500 + d, dtype)
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, heads)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v).cpu().numpy()
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= _tol(dtype)
    st.free()
    idx.free()


@pytest.mark.parametrize("d", [16, 64])
@pytest.mark.parametrize("window", [1, 4])
def test_decode_order5_after_prefill(sata, oracle, d, window):
    n0, T, heads = 70, 9, 2
    x = si.draw_qkv((1, heads), n0 + T, d, d, 5600 + d + window, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("decode P=5 d=%d window %d after %d tokens" % (d, window, n0))
    st = sata.State(idx, 1, heads)
    outs = [prefill(idx, st, q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous())
            .cpu().numpy()]
    sata.sata_state_set_decode_window(st, window)
    outs += [decode(idx, st, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous())
             .cpu().numpy()[:, :, None] for t in range(n0, n0 + T)]
    o = np.concatenate(outs, axis=2)
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= TOL_F32
    st.free()
    idx.free()


def test_decode_order5_bf16_state_matches_emulation(sata, oracle):
    d, n0, T, heads = 16, 64, 40, 2
    x = si.draw_qkv((1, heads), n0 + T, d, d, 5700, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("decode P=5 on a bf16 state d=%d" % d)
    st32 = sata.State(idx, 1, heads)
    prefill(idx, st32, q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous())
    st = sata.State(idx, 1, heads, dtype=torch.bfloat16)
    sata.sata_state_convert(st32, st)
    o = torch.stack([decode(idx, st, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous())
                     for t in range(n0, n0 + T)], dim=2).cpu().numpy()
    ref = oracle.bf16_state_decode(x.q, x.k, x.v, P, n0)
    exact = oracle.taylor_attention(x.q, x.k, x.v, P, rows=np.arange(n0, n0 + T, dtype=np.int64))
    err, drift = rel_err(o, ref), rel_err(ref, exact)
    say("  err vs emulation %.3e, drift %.3e" % (err, drift))
    assert err <= 1e-3 + 1e-2 * drift


@pytest.mark.parametrize("d", [8, 16])
def test_backward_order5(sata, oracle, d):
    n = 150
    x = si.draw_qkv((1, 2), n, d, d, 5800 + d, "f32")
    dout = torch.from_numpy(np.random.default_rng(d).standard_normal((1, 2, n, d)).astype(np.float32)).cuda()
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    grads = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for _ in range(3)]
    say("backward P=5 d=%d" % d)
    sata.sata_prefill_backward(idx, q, k, v, dout, *grads)
    got = [g.cpu().numpy().astype(np.float64) for g in grads]
    ref = oracle.taylor_attention_grad(x.q, x.k, x.v, dout.cpu().numpy(), P)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        a2, b2 = a.reshape(2, -1), np.asarray(b, dtype=np.float64).reshape(2, -1)
        err = float(np.max(np.abs(a2 - b2).max(1) / np.abs(b2).max(1)))
        say("  %s %.3e" % (name, err))
        assert err <= 5e-5
    idx.free()


def test_workload_prefill_d64_p5_bf16_sampled_rows(sata, oracle):
    """1 x 8 heads x 8192 tokens at d = 64, P = 5, bf16: sampled rows of every
    head (the first and last chunks and 64 seeded uniform rows) against O1."""
    wl = si.WORKLOADS["prefill_d64_p5_bf16"]
    say("workload %s" % wl.name)
    x = wl.draw()
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v, chunk=wl.chunk).cpu().numpy()
    rows = sample_rows(wl.n, wl.chunk, 64, 12)
    ref = oracle.taylor_attention(x.q, x.k, x.v, wl.P, rows=rows)
    err = rel_err(o[:, :, rows], ref)
    say("  err %.3e over %d rows x %d heads" % (err, len(rows), wl.heads))
    assert err <= TOL_BF16
    st.free()
    idx.free()


def test_prefill_in_two_segments_sampled_rows(sata, oracle):
    """1 x 16 heads x 8192 tokens at d = 64, P = 5, bf16: the readout partials
    (about 30 GB) exceed the 16 GB workspace cap, so the call runs as two
    segments, the second continuing the state the first left; sampled rows of
    every head against O1."""
    d, heads, n = 64, 16, 8192
    say("prefill P=5 d=64 1x%d heads n=%d (two segments)" % (heads, n))
    x = si.draw_qkv((1, heads), n, d, d, 5900, "bf16")
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, heads)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v, chunk=128).cpu().numpy()
    rows = sample_rows(n, 128, 48, 13)
    err = rel_err(o[:, :, rows], oracle.taylor_attention(x.q, x.k, x.v, P, rows=rows))
    say("  err %.3e over %d rows x %d heads" % (err, len(rows), heads))
    assert err <= TOL_BF16
    del q, k, v
    st.free()
    idx.free()
    torch.cuda.empty_cache()
