"""Head size 128 (d_K = d_V = 128): the table-driven kernels (expansion, the
row-split decode step and read kernel, the matrix-core fold, the finish
kernel), the chunked fp16-operand prefill scan (bf16 inputs, P <= 4: 64-token
chunks, one position per update wavefront) and the block prefill for the rest
(fp32 inputs: blocks of up to 64 tokens read out against the state in HBM,
direct terms inside the block, then folded in) against the oracle; the
backward for bf16 inputs and 3 <= P <= 4 (every pass on the fp16-operand
scan) against the oracle's gradients, and its refusal otherwise."""
import math

import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import TOL_BF16, TOL_F32, decode, dev_all, prefill, rel_err, sample_rows, say

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as s
    s.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return s


def _steps(idx, st, x, lo, hi):
    q, k, v = dev_all(x)
    outs = [decode(idx, st, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous())
            for t in range(lo, hi)]
    return torch.stack(outs, dim=2).cpu().numpy()


def test_expand_d128_matches_bruteforce_basis(sata, oracle):
    P = 3
    say("expand d=128 P=3")
    idx = sata.Index(D, D, P)
    x = si.draw_qkv((1,), 5, D, D, 8800, "f32").q[0]
    xt = torch.from_numpy(x).cuda()
    outs = []
    for side in (0, 1):
        o = torch.zeros((5, idx.m_pad), dtype=torch.float32, device="cuda")
        sata.sata_expand_features(idx, xt, o, side)
        outs.append(o.cpu().numpy().astype(np.float64))
    xd = x.astype(np.float64)
    f = 0
    for p in range(P):
        tup, cnt = oracle.basis_bruteforce(D, p)
        mono = np.prod(xd[:, tup], axis=-1) if p else np.ones((5, 1))
        w = cnt / (math.factorial(p) * math.sqrt(D) ** p)
        g = len(cnt)
        np.testing.assert_allclose(outs[0][:, f:f + g], mono, rtol=4e-7, atol=1e-30)
        np.testing.assert_allclose(outs[1][:, f:f + g], mono * w, rtol=8e-7, atol=1e-30)
        f += g
    assert f == idx.m
    idx.free()


@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_decode_d128_from_empty_every_row(sata, oracle, P):
    n, heads = 20, 2
    x = si.draw_qkv((1, heads), n, D, D, 8900 + P, "f32")
    idx = sata.Index(D, D, P)
    say("decode d=128 P=%d, %d steps from empty" % (P, n))
    st = sata.State(idx, 1, heads)
    o = _steps(idx, st, x, 0, n)
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= TOL_F32
    st.free()
    idx.free()


@pytest.mark.parametrize("window,n", [(4, 23), (64, 70)])
def test_decode_d128_window(sata, oracle, window, n):
    P, heads = 4, 2
    x = si.draw_qkv((1, heads), n, D, D, 9000 + window, "f32")
    idx = sata.Index(D, D, P)
    say("decode d=128 window %d, %d steps" % (window, n))
    st = sata.State(idx, 1, heads)
    sata.sata_state_set_decode_window(st, window)
    o = _steps(idx, st, x, 0, n)
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= TOL_F32
    st.free()
    idx.free()


def test_decode_d128_bf16_state_matches_emulation(sata, oracle):
    P, n, heads = 3, 30, 2
    x = si.draw_qkv((1, heads), n, D, D, 9100, "f32")
    idx = sata.Index(D, D, P)
    say("decode d=128 on a bf16 state, %d steps" % n)
    st = sata.State(idx, 1, heads, dtype=torch.bfloat16)
    o = _steps(idx, st, x, 0, n)
    ref = oracle.bf16_state_decode(x.q, x.k, x.v, P, 0)
    exact = oracle.taylor_attention(x.q, x.k, x.v, P)
    err, drift = rel_err(o, ref), rel_err(ref, exact)
    say("  err vs emulation %.3e, drift %.3e" % (err, drift))
    assert err <= 1e-3 + 1e-2 * drift
    st.free()
    idx.free()


@pytest.mark.parametrize("P,dtype", [(4, "f32"), (2, "f32"), (4, "bf16")])
def test_prefill_d128_every_row(sata, oracle, P, dtype):
    n, heads = 150, 2                                    # blocks of 64, 64 and 22 tokens
    x = si.draw_qkv((1, heads), n, D, D, 9200 + P, dtype)
    idx = sata.Index(D, D, P)
    say("prefill d=128 P=%d %s n=%d" % (P, dtype, n))
    st = sata.State(idx, 1, heads)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v).cpu().numpy()
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    st.free()
    idx.free()


@pytest.mark.parametrize("P", [2, 3, 4])
def test_prefill_d128_chunked_every_row(sata, oracle, P):
    """Chunked scan: four 64-token chunks and a ragged 37, every row against O1; then two
    decode steps continue from the state the scan left."""
    n, t, heads = 4 * 64 + 37, 2, 2
    x = si.draw_qkv((1, heads), n + t, D, D, 9400 + P, "bf16")
    plan = sata.sata_describe_prefill_plan(D, P, heads, n, 0, sata.SATA_BF16)
    say("prefill d=128 chunked P=%d bf16 n=%d: %d slices per head" % (P, n, plan["slices"]))
    idx = sata.Index(D, D, P)
    st = sata.State(idx, 1, heads)
    q, k, v = dev_all(x)
    sl = lambda a, lo, hi: a[:, :, lo:hi].contiguous()
    o = prefill(idx, st, sl(q, 0, n), sl(k, 0, n), sl(v, 0, n)).cpu().numpy()
    ref = oracle.taylor_attention(x.q, x.k, x.v, P)
    err = rel_err(o, ref[:, :, :n])
    say("  prefill err %.3e; decode %d steps" % (err, t))
    assert err <= TOL_BF16
    od = _steps(idx, st, x, n, n + t)
    errd = rel_err(od, ref[:, :, n:])
    say("  decode err %.3e" % errd)
    assert errd <= TOL_BF16
    st.free()
    idx.free()


def test_prefill_d128_chunked_workload_sampled_rows(sata, oracle):
    """The 1 x 8 x 4096 bf16 workload at P = 4 (1,430 slices per head, one segment): the
    first and last chunk and 64 seeded rows of every head against O1."""
    wl = si.WORKLOADS["prefill_d128_p4_bf16"]
    x = wl.draw()
    say("prefill %s" % wl.name)
    idx = sata.Index(D, D, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v, chunk=wl.chunk).cpu().numpy()
    rows = sample_rows(wl.n, wl.chunk, 64, wl.seed + 1)
    ref = oracle.taylor_attention(x.q, x.k, x.v, wl.P, rows=rows)
    err = rel_err(o[:, :, rows], ref)
    say("  %d rows x %d heads: err %.3e" % (len(rows), wl.heads, err))
    assert err <= TOL_BF16
    st.free()
    idx.free()


def test_prefill_d128_continued_by_decode_and_prefill(sata, oracle):
    """prefill 70, decode 5 at window 4 (one token left pending), prefill 30
    (folds it first), decode 3: every row against O1."""
    P, heads, n1, t1, n2, t2 = 3, 2, 70, 5, 30, 3
    n = n1 + t1 + n2 + t2
    x = si.draw_qkv((1, heads), n, D, D, 9300, "f32")
    idx = sata.Index(D, D, P)
    q, k, v = dev_all(x)
    sl = lambda a, lo, hi: a[:, :, lo:hi].contiguous()
    say("prefill/decode interleaved d=128, n=%d" % n)
    st = sata.State(idx, 1, heads)
    outs = [prefill(idx, st, sl(q, 0, n1), sl(k, 0, n1), sl(v, 0, n1)).cpu().numpy()]
    sata.sata_state_set_decode_window(st, 4)
    outs.append(_steps(idx, st, x, n1, n1 + t1))
    p0 = n1 + t1
    outs.append(prefill(idx, st, sl(q, p0, p0 + n2), sl(k, p0, p0 + n2), sl(v, p0, p0 + n2)).cpu().numpy())
    outs.append(_steps(idx, st, x, p0 + n2, n))
    err = rel_err(np.concatenate(outs, axis=2), oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= TOL_F32
    st.free()
    idx.free()


@pytest.mark.parametrize("P", [3, 4])
def test_d128_backward_bf16(sata, oracle, P):
    """dq, dk, dv of a ragged bf16 prefill (two 64-token chunks and 22) on two heads against
    O9, normwise per head; a second call on the same index (its P - 1 order index is then
    reused) gives the same bits."""
    n, heads = 150, 2
    x = si.draw_qkv((1, heads), n, D, D, 9500 + P, "bf16")
    dout = np.random.default_rng(9510 + P).standard_normal((1, heads, n, D)).astype(np.float32)
    idx = sata.Index(D, D, P)
    q, k, v = dev_all(x)
    do = torch.from_numpy(dout).cuda().to(torch.bfloat16)
    say("backward d=128 P=%d bf16 n=%d" % (P, n))
    runs = []
    for _ in range(2):
        g = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for _ in range(3)]
        sata.sata_prefill_backward(idx, q, k, v, do, *g)
        torch.cuda.synchronize()
        runs.append(g)
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    ref = oracle.taylor_attention_grad(x.q, x.k, x.v, do.float().cpu().numpy(), P)
    for name, a, r in zip(("dq", "dk", "dv"), runs[0], ref):
        a = a.cpu().numpy().astype(np.float64)
        err = float((np.abs(a - r).reshape(heads, -1).max(1) / np.abs(r).reshape(heads, -1).max(1)).max())
        say("  %s err %.3e" % (name, err))
        assert err <= TOL_BF16, name
    idx.free()


@pytest.mark.parametrize("P,dtype", [(3, torch.float32), (2, torch.bfloat16)])
def test_d128_backward_refused(sata, P, dtype):
    """fp32 inputs (no chunked scan at this head size) and P = 2 (whose dk and dq passes have
    order 0 alone, outside the fp16-operand scan) are refused before any work."""
    idx = sata.Index(D, D, P)
    q = torch.zeros((1, 1, 8, D), device="cuda", dtype=dtype)
    g = [torch.zeros_like(q) for _ in range(3)]
    with pytest.raises(sata.SataError) as e:
        sata.sata_prefill_backward(idx, q, q, q, q, g[0], g[1], g[2])
    assert e.value.status == sata.SATA_ERR_UNSUPPORTED
    idx.free()
