"""GPU parity of the prefill backward (dq, dk, dv through the C ABI) against the
oracle's gradients of the quadratic definition (O9).

Metric, per head and gradient: max |g - g_ref| / max |g_ref| (normwise over
the head's whole gradient: single rows of dq or dk can be near zero).  Bars:
TOL_GRAD_F32 for fp32 inputs (the passes run the fp32 prefill path; the
gradients are sums of a few of its results, so a few times its 1e-5), and
the bf16-input bar for bf16 inputs (the passes also round their values,
g_i[c] q_i and [v_j, 1][c] k_j: to binary16 on the fp16-operand scan, which
takes every pass whose head size and order it covers, else to bf16).
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import TOL_BF16, dev, say

pytestmark = pytest.mark.gpu

TOL_GRAD_F32 = 5e-5


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as s
    s.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return s


def grad_err(a, ref) -> float:
    a = np.asarray(a, dtype=np.float64).reshape(-1, *ref.shape[-2:])
    ref = np.asarray(ref, dtype=np.float64).reshape(a.shape)
    num = np.abs(a - ref).reshape(a.shape[0], -1).max(1)
    den = np.abs(ref).reshape(a.shape[0], -1).max(1)
    return float(np.max(num / np.maximum(den, 1e-300)))


def _run(sata, idx, x, dout, chunk=0, grad_dtype=torch.float32):
    q, k, v = dev(x, "q"), dev(x, "k"), dev(x, "v")
    do = dout.to(q.dtype)
    dq, dk, dv = (torch.empty(q.shape, dtype=grad_dtype, device="cuda") for _ in range(3))
    sata.sata_prefill_backward(idx, q, k, v, do, dq, dk, dv, chunk=chunk)
    return [t.float().cpu().numpy() for t in (dq, dk, dv)], do.float().cpu().numpy()


def _check(oracle, x, do_np, P, got, tol, label):
    ref = oracle.taylor_attention_grad(x.q, x.k, x.v, do_np, P)
    errs = [grad_err(a, b) for a, b in zip(got, ref)]
    say("  %s: dq %.3e  dk %.3e  dv %.3e" % (label, *errs))
    assert max(errs) <= tol, errs


@pytest.mark.parametrize("d", [8, 16, 32, 64])
@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_backward_all_shapes_ragged(sata, oracle, d, P):
    n = 150                                      # two chunks of 64 and a ragged tail
    x = si.draw_qkv((1, 2), n, d, d, 4000 + 10 * d + P, "f32")
    dout = torch.from_numpy(np.random.default_rng(d + P).standard_normal((1, 2, n, d)).astype(np.float32)).cuda()
    idx = sata.Index(d, d, P)
    say("backward d=%d P=%d n=%d" % (d, P, n))
    got, do_np = _run(sata, idx, x, dout)
    _check(oracle, x, do_np, P, got, TOL_GRAD_F32, "fp32")


def test_backward_bf16_inputs(sata, oracle):
    d, P, n = 32, 4, 200
    x = si.draw_qkv((2, 2), n, d, d, 4100, "bf16")
    dout = torch.from_numpy(np.random.default_rng(7).standard_normal((2, 2, n, d)).astype(np.float32)).cuda()
    idx = sata.Index(d, d, P)
    say("backward bf16 d=%d n=%d" % (d, n))
    got, do_np = _run(sata, idx, x, dout, grad_dtype=torch.bfloat16)
    _check(oracle, x, do_np, P, got, TOL_BF16, "bf16")


def test_backward_chunk_invariance(sata, oracle):
    d, P, n = 16, 4, 300
    x = si.draw_qkv((1, 3), n, d, d, 4200, "f32")
    dout = torch.from_numpy(np.random.default_rng(8).standard_normal((1, 3, n, d)).astype(np.float32)).cuda()
    idx = sata.Index(d, d, P)
    say("backward chunk 64 vs 128")
    a, _ = _run(sata, idx, x, dout, chunk=64)
    b, do_np = _run(sata, idx, x, dout, chunk=128)
    for u, w in zip(a, b):
        assert grad_err(u, w) <= TOL_GRAD_F32
    _check(oracle, x, do_np, P, b, TOL_GRAD_F32, "chunk 128")


def test_backward_workload_d16_f32(sata, oracle):
    """1 x 8 heads, n = 4096, d = 16, P = 4, fp32: every head against O9."""
    wl = si.WORKLOADS["prefill_d16_p4_f32"]
    x = wl.draw()
    dout = torch.from_numpy(np.random.default_rng(9).standard_normal(x.q.shape[:-1] + (wl.d_v,))
                            .astype(np.float32)).cuda()
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    say("backward workload %s" % wl.name)
    got, do_np = _run(sata, idx, x, dout)
    _check(oracle, x, do_np, wl.P, got, TOL_GRAD_F32, wl.name)


def test_backward_d64_bf16_workload_heads(sata, oracle):
    """The d_K = 64, P = 4 bf16 workload's head count (1 x 8) on 8192 tokens (the oracle's
    n x n weights bound n), two heads against O9."""
    d, P, n = 64, 4, 8192
    x = si.draw_qkv((1, 8), n, d, d, 4646, "bf16")
    dout = torch.from_numpy(np.random.default_rng(4647).standard_normal((1, 8, n, d)).astype(np.float32)).cuda()
    idx = sata.Index(d, d, P)
    say("backward bf16 d=64 P=4, 1 x 8 heads x %d tokens" % n)
    got, do_np = _run(sata, idx, x, dout, chunk=128)
    hs = [0, 7]
    sub = lambda a: np.ascontiguousarray(a[:, hs])
    xs = si.QKV(sub(x.q), sub(x.k), sub(x.v), "f32")
    _check(oracle, xs, sub(do_np), P, [sub(g) for g in got], TOL_BF16, "heads 0, 7")
    idx.free()


def test_backward_d64_bf16_workload_full_size(sata):
    """The full d_K = 64 workload (1 x 8 heads x 65536 tokens, bf16), whose passes plan
    workspaces near the 16 GB cap, where O9 cannot run: properties that hold at any size.
    Every pass is linear in dout, and the gradient-weighted values enter the passes scaled by
    a power of two chosen from the largest |g|, which doubling dout halves: the passes see the
    same bits, and doubling dout doubles every gradient bit for bit.  The attention weights of
    each query sum to one, so sum_j dv_j = sum_i dout_i (normwise within the bf16-input bar)."""
    wl = si.WORKLOADS["prefill_d64_p4_bf16"]
    say("backward full size %s" % wl.name)
    q, k, v = si.draw_qkv_device((wl.batch, wl.heads), wl.n, wl.d_k, wl.d_v, wl.seed, "bf16")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4648)
    do = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    grads = []
    for scale in (1.0, 2.0):
        g = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for _ in range(3)]
        sata.sata_prefill_backward(idx, q, k, v, (do.float() * scale).to(torch.bfloat16), *g, chunk=wl.chunk)
        torch.cuda.synchronize()
        grads.append(g)
    for name, a, b in zip(("dq", "dk", "dv"), grads[0], grads[1]):
        assert torch.isfinite(a).all(), name
        say("  %s: doubling dout doubles it exactly: %s" % (name, bool(torch.equal(b, 2 * a))))
        assert torch.equal(b, 2 * a), name
    dv_sum = grads[0][2].double().sum(dim=2)                  # [B, H, d_V]
    do_sum = do.double().sum(dim=2)
    err = float(((dv_sum - do_sum).abs().amax(-1) / do_sum.abs().amax(-1)).max())
    say("  sum dv vs sum dout: %.3e" % err)
    assert err <= TOL_BF16
    idx.free()


def test_backward_error_paths(sata):
    idx = sata.Index(16, 16, 4)
    q = torch.zeros((1, 1, 8, 16), device="cuda")
    g = [torch.zeros_like(q) for _ in range(3)]
    with pytest.raises(sata.SataError) as e:
        sata.sata_prefill_backward(idx, q, q, q, q, g[0], g[1], g[2], chunk=96)
    assert e.value.status == sata.SATA_ERR_UNSUPPORTED
    with pytest.raises(sata.SataError) as e:
        sata.sata_prefill_backward(idx, q, q, q, q, q, g[1], g[2])     # dq aliases q
    assert e.value.status == sata.SATA_ERR_INVALID
    with pytest.raises(sata.SataError) as e:
        sata.sata_prefill_backward(idx, q, q, q, q, g[0], g[0], g[2])  # dq aliases dk
    assert e.value.status == sata.SATA_ERR_INVALID


def test_backward_temporaries_kept_with_the_index(sata):
    """Backward calls on one index take their temporaries from a pool kept with
    the index: after the first call the device's free memory stays put over
    further calls, with another index created, used for a backward and freed
    between them; the gradients repeat bit for bit; freeing the index returns
    the pool's memory."""
    d, P, n, heads = 64, 4, 1024, 2
    x = si.draw_qkv((1, heads), n, d, d, 4321, "bf16")
    q, k, v = dev(x, "q"), dev(x, "k"), dev(x, "v")
    do = torch.from_numpy(np.random.default_rng(5).standard_normal((1, heads, n, d)).astype(np.float32)).cuda()
    do = do.to(q.dtype)
    grads = [torch.empty(q.shape, dtype=torch.float32, device="cuda") for _ in range(3)]
    xo = si.draw_qkv((1, 1), 200, 32, 32, 4322, "bf16")
    qo, ko, vo = dev(xo, "q"), dev(xo, "k"), dev(xo, "v")
    doo = torch.ones(qo.shape, dtype=qo.dtype, device="cuda")
    go = [torch.empty(qo.shape, dtype=torch.float32, device="cuda") for _ in range(3)]
    idx = sata.Index(d, d, P)
    say("backward pool: %d heads x %d tokens, d=%d" % (heads, n, d))
    sata.sata_prefill_backward(idx, q, k, v, do, *grads)
    torch.cuda.synchronize()
    first = [g.cpu().numpy() for g in grads]
    free_after_first = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        other = sata.Index(32, 32, 4)
        sata.sata_prefill_backward(other, qo, ko, vo, doo, *go)
        other.free()
        sata.sata_prefill_backward(idx, q, k, v, do, *grads)
        torch.cuda.synchronize()
        for a, b in zip(first, grads):
            assert np.array_equal(a, b.cpu().numpy())
        drop = free_after_first - torch.cuda.mem_get_info()[0]
        say("  free memory below the first call's: %.1f MB" % (drop / 2**20))
        assert drop < 64 << 20
    idx.free()
    torch.cuda.synchronize()
    back = torch.cuda.mem_get_info()[0] - free_after_first
    say("  freed with the index: %.1f MB" % (back / 2**20))
    assert back > 0
