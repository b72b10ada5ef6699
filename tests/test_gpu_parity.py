"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Metric: max over rows of ||o - o_oracle||_inf / ||o_oracle||_inf.
Bars: 1e-5 for fp32 inputs, 2e-2 for bf16 inputs (the oracle consumes the
bf16-rounded values, so the bar measures the kernels, not input rounding).
Small cases are checked on every row; the measured workloads at full size on
sampled rows (first and last chunk plus seeded uniform rows).
"""
import math

import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import (TOL_BF16, TOL_F32, decode, dev_all, prefill, rel_err, sample_rows,
                           say)

pytestmark = pytest.mark.gpu

WL = si.WORKLOADS


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as s
    s.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return s


def _tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


# ------------------------------------------------------------------ expansion

@pytest.mark.parametrize("d,P", [(8, 3), (16, 4), (32, 4), (64, 4), (64, 1)])
def test_expand_matches_bruteforce_basis(sata, oracle, d, P):
    """Key side = plain monomial; query side = count/(p! d^(p/2)) * monomial,
    with tuples and counts from the oracle's brute-force enumeration."""
    say("expand d=%d P=%d" % (d, P))
    idx = sata.Index(d, d, P)
    x = si.draw_qkv((1,), 5, d, d, 777 + d, "f32").q[0]          # [5, d]
    xt = torch.from_numpy(x).cuda()
    outs = []
    for side in (0, 1):
        o = torch.zeros((5, idx.m_pad), dtype=torch.float32, device="cuda")
        sata.sata_expand_features(idx, xt, o, side)
        outs.append(o.cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    xd = x.astype(np.float64)
    f = 0
    for p in range(P):
        tup, cnt = oracle.basis_bruteforce(d, p)
        mono = np.prod(xd[:, tup], axis=-1) if p else np.ones((5, 1))
        w = cnt / (math.factorial(p) * math.sqrt(d) ** p)
        g = len(cnt)
        np.testing.assert_allclose(outs[0][:, f:f + g], mono, rtol=4e-7, atol=1e-30)
        np.testing.assert_allclose(outs[1][:, f:f + g], mono * w, rtol=8e-7, atol=1e-30)
        f += g
    assert np.all(outs[0][:, f:] == 0) and np.all(outs[1][:, f:] == 0)
    idx.free()


# ------------------------------------------------------------------ small, every row

def test_tiny_prefill_every_row(sata, oracle):
    wl = WL["tiny_d8_p3"]
    say("prefill %s" % wl.name)
    x = wl.draw()
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v, chunk=wl.chunk).cpu().numpy()
    ref = oracle.taylor_attention(x.q, x.k, x.v, wl.P)
    err = rel_err(o, ref)
    say("  err %.3e" % err)
    assert err <= TOL_F32


def test_tiny_decode_from_empty_state_every_row(sata, oracle):
    """n decode steps from an empty state reproduce the whole causal output."""
    wl = WL["tiny_d8_p3"]
    say("decode-from-empty %s" % wl.name)
    x = wl.draw()
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    q, k, v = dev_all(x)
    outs = []
    for t in range(wl.n):
        outs.append(decode(idx, st, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous()))
    o = torch.stack(outs, dim=2).cpu().numpy()
    ref = oracle.taylor_attention(x.q, x.k, x.v, wl.P)
    err = rel_err(o, ref)
    say("  err %.3e" % err)
    assert err <= TOL_F32


@pytest.mark.parametrize("d", [8, 16, 32, 64])
@pytest.mark.parametrize("P", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_shapes_ragged_every_row(sata, oracle, d, P, dtype):
    """Every supported (d, P), both input dtypes, n = 2 chunks + a ragged tail."""
    chunk = 128 if d == 64 else 64
    n = 2 * chunk + 37
    say("prefill d=%d P=%d %s n=%d" % (d, P, dtype, n))
    x = si.draw_qkv((2, 3), n, d, d, 4242 + 10 * d + P, dtype)
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 2, 3)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v).cpu().numpy()
    ref = oracle.taylor_attention(x.q, x.k, x.v, P)
    err = rel_err(o, ref)
    say("  err %.3e" % err)
    assert err <= _tol(dtype)


@pytest.mark.parametrize("d", [8, 16, 32, 64])
@pytest.mark.parametrize("heads", [1, 64])
@pytest.mark.parametrize("chunk", [64, 128])
def test_bf16_eight_wave_shapes_every_row(sata, oracle, d, heads, chunk):
    """bf16 inputs run on eight wavefronts per workgroup (d_K = 64 in 128-token chunks: every
    wavefront reads out and updates; otherwise readout and update wavefronts apart).  Few heads
    give the smaller slices, many heads the larger; n = 2 chunks + a ragged tail, every row."""
    P = 4
    n = 2 * chunk + 45
    say("prefill bf16 chunk %d d=%d heads=%d n=%d" % (chunk, d, heads, n))
    x = si.draw_qkv((1, heads), n, d, d, 5151 + d + heads, "bf16")
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, heads)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v, chunk=chunk).cpu().numpy()
    err = rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P))
    say("  err %.3e" % err)
    assert err <= TOL_BF16


# bf16 inputs with d_K = d_V in {16, 32, 64}, P <= 4 run the fp16-operand scan, whose update
# wavefronts hold the largest number of positions their registers allow (5, 3, 2 at d = 16, 32,
# 64) unless that leaves fewer (head, slice) work items than compute units; then one.  The
# planned slice count shows which ran: (d, heads, slices).
@pytest.mark.parametrize("d,heads,slices", [(16, 320, 1), (16, 4, 5), (32, 32, 10), (32, 4, 30),
                                            (64, 4, 102), (64, 1, 204)])
def test_fp16_scan_both_slice_widths(sata, oracle, d, heads, slices):
    P, chunk = 4, 128
    n = 2 * chunk + 45
    plan = sata.sata_describe_prefill_plan(d, P, heads, n, chunk, sata.SATA_BF16)
    say("prefill bf16 d=%d heads=%d n=%d: %d slices per head" % (d, heads, n, plan["slices"]))
    assert plan["slices"] == slices
    x = si.draw_qkv((1, heads), n, d, d, 5353 + d + heads, "bf16")
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, heads)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v, chunk=chunk).cpu().numpy()
    hs = sorted({0, min(1, heads - 1), heads // 2, heads - 1})
    sub = lambda a: np.ascontiguousarray(a[:, hs])
    err = rel_err(o[:, hs], oracle.taylor_attention(sub(x.q), sub(x.k), sub(x.v), P))
    say("  heads %s: err %.3e" % (hs, err))
    assert err <= TOL_BF16


@pytest.mark.parametrize("d,chunk", [(16, 128), (32, 128), (64, 128), (16, 0)])
@pytest.mark.parametrize("refresh", [1, 2, 3, 5])
def test_copy_refresh_intervals_every_row(sata, oracle, d, chunk, refresh):
    """The fp16-operand scan rewrites the readout's state copy every `refresh`
    chunks and the reduce kernel adds the keys since the last copy as direct
    terms: every row of a two-call prefill (the second continuing the first's
    state, so the order-0 prefix and the state both carry over) on a ragged
    length matches the oracle at each forced interval, including intervals
    that do not divide the chunk count; chunk 0 at d = 16 is the default
    256-token chunk."""
    P, heads = 4, 3
    n1, n2 = 300, 6 * 128 + 45
    n = n1 + n2
    x = si.draw_qkv((1, heads), n, d, d, 8080 + d + refresh, "bf16")
    ref = oracle.taylor_attention(x.q, x.k, x.v, P)
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, heads)
    q, k, v = dev_all(x)
    say("prefill bf16 d=%d chunk %d refresh %d: %d + %d tokens" % (d, chunk, refresh, n1, n2))
    try:
        sata.sata_debug_prefill_refresh(refresh)
        part = lambda a, lo, hi: a[:, :, lo:hi].contiguous()
        o1 = prefill(idx, st, part(q, 0, n1), part(k, 0, n1), part(v, 0, n1), chunk=chunk)
        o2 = prefill(idx, st, part(q, n1, n), part(k, n1, n), part(v, n1, n), chunk=chunk)
    finally:
        sata.sata_debug_prefill_refresh(0)
    o = torch.cat([o1, o2], dim=2).cpu().numpy()
    err = rel_err(o, ref)
    say("  err %.3e" % err)
    assert err <= TOL_BF16


def test_short_sequences_and_empty(sata, oracle):
    d, P = 16, 4
    idx = sata.Index(d, d, P)
    for n in (1, 5, 63, 64, 65):
        say("prefill short n=%d" % n)
        x = si.draw_qkv((1, 2), n, d, d, 99 + n, "f32")
        st = sata.State(idx, 1, 2)
        q, k, v = dev_all(x)
        o = prefill(idx, st, q, k, v).cpu().numpy()
        assert rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P)) <= TOL_F32
    # n = 0 is a no-op and leaves the state untouched
    st = sata.State(idx, 1, 2)
    e = torch.empty((1, 2, 0, d), device="cuda")
    sata.sata_prefill(idx, st, e, e, e, torch.empty((1, 2, 0, d), device="cuda"))
    assert float(sata.state_tensor(st).abs().max()) == 0.0


def test_chunk_length_invariance(sata, oracle):
    d, P, n = 32, 4, 3 * 128 + 11
    x = si.draw_qkv((1, 4), n, d, d, 31337, "f32")
    ref = oracle.taylor_attention(x.q, x.k, x.v, P)
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    res = {}
    for chunk in (64, 128):
        say("chunk invariance chunk=%d" % chunk)
        st = sata.State(idx, 1, 4)
        res[chunk] = prefill(idx, st, q, k, v, chunk=chunk).cpu().numpy()
        assert rel_err(res[chunk], ref) <= TOL_F32
    assert rel_err(res[64], res[128]) <= 2 * TOL_F32


def test_split_prefill_and_decode_continuation(sata, oracle):
    """prefill(n1) then prefill(n2) then t decode steps == the causal output of
    the whole sequence (the state carries everything)."""
    d, P, n1, n2, t = 16, 4, 100, 157, 9
    n = n1 + n2 + t
    x = si.draw_qkv((2, 2), n, d, d, 2024, "f32")
    ref = oracle.taylor_attention(x.q, x.k, x.v, P)
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 2, 2)
    q, k, v = dev_all(x)
    say("split prefill %d + %d + %d decode" % (n1, n2, t))
    o1 = prefill(idx, st, q[:, :, :n1].contiguous(), k[:, :, :n1].contiguous(), v[:, :, :n1].contiguous())
    o2 = prefill(idx, st, q[:, :, n1:n1 + n2].contiguous(), k[:, :, n1:n1 + n2].contiguous(),
                 v[:, :, n1:n1 + n2].contiguous())
    o3 = [decode(idx, st, q[:, :, i].contiguous(), k[:, :, i].contiguous(), v[:, :, i].contiguous())
          for i in range(n1 + n2, n)]
    o = torch.cat([o1, o2, torch.stack(o3, dim=2)], dim=2).cpu().numpy()
    assert rel_err(o, ref) <= TOL_F32


def test_state_content_matches_definition(sata):
    """After a prefill, state row c of feature f = sum_s prod_r k_s[i_r] * [v_s, 1][c]
    (fp64 reference from the library's own tuple description)."""
    d, P, n = 8, 3, 150
    x = si.draw_qkv((1, 1), n, d, d, 555, "f32")
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, 1)
    q, k, v = dev_all(x)
    say("state content d=%d" % d)
    prefill(idx, st, q, k, v)
    S = sata.state_tensor(st).cpu().numpy()[0, 0].astype(np.float64)      # [d+1, m_pad]
    tup, _ = sata.sata_describe_features(d, P)
    kk = np.concatenate([x.k[0, 0].astype(np.float64), np.ones((n, 1)), np.zeros((n, 1))], axis=1)
    slots = np.stack([(tup >> (8 * r)) & 0xFF for r in range(3)], axis=1).astype(np.int64)
    mono = kk[:, slots[:, 0]] * kk[:, slots[:, 1]] * kk[:, slots[:, 2]]   # [n, m]
    vext = np.concatenate([x.v[0, 0].astype(np.float64), np.ones((n, 1))], axis=1)
    ref = vext.T @ mono                                                    # [d+1, m]
    m = len(tup)
    np.testing.assert_allclose(S[:, :m], ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
    assert np.all(S[:, m:] == 0)


def test_many_heads_subsegment_handoff(sata, oracle):
    """320 heads x 4096 tokens (d=16, fp32, chunk 128): more scan work items
    than CUs, so each slice's 32 chunks run as two sub-segments whose state
    is handed over through memory between workgroups.  Sampled rows of four
    heads and two decode steps that continue from the handed-over state are
    held to the fp32 bar."""
    d, P, n, t, nh = 16, 4, 4096, 2, 320
    x = si.draw_qkv((1, nh), n + t, d, d, 4242, "f32")
    heads = [0, 101, 202, nh - 1]
    rows = sample_rows(n, 128, 48, 77)
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, nh)
    q, k, v = dev_all(x)
    say("sub-segment handoff: %d heads x %d tokens" % (nh, n))
    o = prefill(idx, st, q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous(), chunk=128)
    od = [decode(idx, st, q[:, :, i].contiguous(), k[:, :, i].contiguous(), v[:, :, i].contiguous())
          for i in range(n, n + t)]
    got = o.cpu().numpy()[:, heads][:, :, rows]
    sub = lambda a: np.ascontiguousarray(a[:, heads])
    ref = oracle.taylor_attention(sub(x.q), sub(x.k), sub(x.v), P, rows=np.concatenate([rows, np.arange(n, n + t)]))
    err = rel_err(got, ref[:, :, :len(rows)])
    gotd = torch.stack(od, dim=2).cpu().numpy()[:, heads]
    errd = rel_err(gotd, ref[:, :, len(rows):])
    say("  err %.3e, decode err %.3e" % (err, errd))
    assert err <= TOL_F32 and errd <= TOL_F32


def test_deterministic_and_checkpoint_restore(sata):
    d, P, n = 32, 4, 300
    x = si.draw_qkv((2, 2), n + 4, d, d, 8080, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("determinism + checkpoint")
    a = sata.State(idx, 2, 2)
    b = sata.State(idx, 2, 2)
    oa = prefill(idx, a, q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous())
    ob = prefill(idx, b, q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous())
    assert torch.equal(oa, ob)
    assert torch.equal(sata.state_tensor(a), sata.state_tensor(b))
    snap = sata.state_tensor(a).clone()
    steps = [(q[:, :, i].contiguous(), k[:, :, i].contiguous(), v[:, :, i].contiguous()) for i in range(n, n + 4)]
    first = [decode(idx, a, *s) for s in steps]
    sata.state_tensor(a).copy_(snap)
    second = [decode(idx, a, *s) for s in steps]
    for u, w in zip(first, second):
        assert torch.equal(u, w)


def test_nan_in_one_head_does_not_leak(sata):
    d, P, n = 16, 4, 130
    x = si.draw_qkv((1, 4), n, d, d, 6060, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("nan isolation")
    clean = prefill(idx, sata.State(idx, 1, 4), q, k, v)
    v2 = v.clone()
    v2[0, 2, 17, 3] = float("nan")
    dirty = prefill(idx, sata.State(idx, 1, 4), q, k, v2)
    for h in (0, 1, 3):
        assert torch.equal(clean[0, h], dirty[0, h])
    assert torch.isnan(dirty[0, 2, 17:]).any()


def test_bf16_output(sata, oracle):
    d, P, n = 32, 4, 200
    x = si.draw_qkv((1, 2), n, d, d, 1212, "bf16")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("bf16 output")
    o = prefill(idx, sata.State(idx, 1, 2), q, k, v, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert rel_err(o, oracle.taylor_attention(x.q, x.k, x.v, P)) <= TOL_BF16


def test_error_paths(sata):
    idx = sata.Index(16, 16, 4)
    st = sata.State(idx, 1, 1)
    q = torch.zeros((1, 1, 8, 16), device="cuda")
    with pytest.raises(sata.SataError) as e:
        sata.sata_prefill(idx, st, q, q, q, torch.zeros_like(q), chunk=96)
    assert e.value.status == sata.SATA_ERR_UNSUPPORTED
    with pytest.raises(sata.SataError) as e:
        sata.sata_prefill(idx, st, q, q, q, q)                  # out aliases q
    assert e.value.status == sata.SATA_ERR_INVALID
    lib = sata.load()
    base = torch.zeros(64, device="cuda")
    mis = base.data_ptr() + 4
    rc = lib.sata_prefill(idx.ptr, st.ptr, mis, mis, mis, base.data_ptr() + 128, 1, 0, 0, 0, None)
    assert rc == sata.SATA_ERR_INVALID
    other = sata.Index(16, 16, 3)
    with pytest.raises(sata.SataError):
        sata.sata_prefill(other, st, q, q, q, torch.zeros_like(q))


# ------------------------------------------------------------------ measured workloads, full size

def _prefill_workload(sata, oracle, wl, extra_rows):
    say("prefill workload %s" % wl.name)
    x = wl.draw()
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    q, k, v = dev_all(x)
    o = prefill(idx, st, q, k, v, chunk=wl.chunk)
    torch.cuda.synchronize()
    # (chunk 0, the default, is 256 tokens where it is used here: the d = 16 fp16-operand scan)
    rows = None if extra_rows is None else sample_rows(wl.n, wl.chunk or 256, extra_rows, wl.seed)
    o = o.cpu().numpy()
    ref = oracle.taylor_attention(x.q, x.k, x.v, wl.P, rows=rows)
    got = o if rows is None else o[:, :, rows]
    err = rel_err(got, ref)
    say("  err %.3e over %s rows" % (err, "all" if rows is None else len(rows)))
    return err


def test_workload_prefill_d16_f32_every_row(sata, oracle):
    assert _prefill_workload(sata, oracle, WL["prefill_d16_p4_f32"], None) <= TOL_F32


def test_workload_prefill_d32_bf16_sampled(sata, oracle):
    assert _prefill_workload(sata, oracle, WL["prefill_d32_p4_bf16"], 128) <= TOL_BF16


def test_workload_prefill_d64_bf16_sampled(sata, oracle):
    assert _prefill_workload(sata, oracle, WL["prefill_d64_p4_bf16"], 64) <= TOL_BF16


def test_workload_prefill_d16x64h_bf16_sampled(sata, oracle):
    assert _prefill_workload(sata, oracle, WL["prefill_d16x64h_p4_bf16"], 32) <= TOL_BF16


def test_workload_prefill_d16x64h_default_chunk_sampled(sata, oracle):
    """The same workload at the library's default chunk for this head size (256 tokens): 512
    chunks per head in sub-segments, sampled rows of every head against the oracle."""
    import dataclasses
    wl = dataclasses.replace(WL["prefill_d16x64h_p4_bf16"], chunk=0)
    plan = sata.sata_describe_prefill_plan(wl.d_k, wl.P, wl.batch * wl.heads, wl.n, 0, sata.SATA_BF16)
    say("default chunk plan: %s" % plan)
    assert plan["seg_chunks"] * 256 >= wl.n            # one segment of 256-token chunks
    assert _prefill_workload(sata, oracle, wl, 32) <= TOL_BF16


def test_workload_decode_d64_after_8192(sata, oracle):
    """32 x 8 heads, state built by an fp32 prefill of 8192 tokens, then decode
    steps with fresh inputs; every head of every step against the oracle."""
    wl = WL["decode_d64_p4_f32"]
    steps = 6
    say("decode workload %s (%d steps)" % (wl.name, steps))
    pre = wl.draw()
    dec = wl.draw_decode(steps)
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    q, k, v = dev_all(pre)
    prefill(idx, st, q, k, v)
    del q, k, v
    dq, dk_, dv_ = dev_all(dec)
    outs = [decode(idx, st, dq[:, :, t].contiguous(), dk_[:, :, t].contiguous(), dv_[:, :, t].contiguous())
            for t in range(steps)]
    o = torch.stack(outs, dim=2).cpu().numpy()
    qa = np.concatenate([pre.q, dec.q], axis=2)
    ka = np.concatenate([pre.k, dec.k], axis=2)
    va = np.concatenate([pre.v, dec.v], axis=2)
    rows = np.arange(wl.n, wl.n + steps, dtype=np.int64)
    ref = oracle.taylor_attention(qa, ka, va, wl.P, rows=rows)
    err = rel_err(o, ref)
    say("  err %.3e" % err)
    assert err <= TOL_F32


def test_workload_decode_d64_all_1024_steps(sata, oracle):
    """The decode workload as configured: 32 x 8 heads, an fp32 prefill of 8192
    tokens, then all 1024 recurrent decode steps with fresh inputs.  Every step
    of eight heads spread over the batch (entries 0, 9, 22 and 31) is held to
    the fp32 bar against the oracle's rows 8192 .. 9215, so drift of the
    state over the full run of read-modify-write steps would show."""
    wl = WL["decode_d64_p4_f32"]
    steps = 1024
    say("decode workload %s, all %d steps" % (wl.name, steps))
    pre = wl.draw()
    dec = wl.draw_decode(steps)
    idx = sata.Index(wl.d_k, wl.d_v, wl.P)
    st = sata.State(idx, wl.batch, wl.heads)
    q, k, v = dev_all(pre)
    prefill(idx, st, q, k, v)
    del q, k, v
    dq, dk_, dv_ = dev_all(dec)
    o = torch.empty((wl.batch, wl.heads, steps, wl.d_v), device="cuda")
    for t in range(steps):
        o[:, :, t] = decode(idx, st, dq[:, :, t].contiguous(), dk_[:, :, t].contiguous(), dv_[:, :, t].contiguous())
    torch.cuda.synchronize()
    picks = [(0, 0), (0, 7), (9, 3), (9, 4), (22, 1), (22, 6), (31, 0), (31, 7)]
    got = np.stack([o[b, h].cpu().numpy() for b, h in picks])[None]
    cat = lambda a, b: np.stack([np.concatenate([a[bb, hh], b[bb, hh]]) for bb, hh in picks])[None]
    rows = np.arange(wl.n, wl.n + steps, dtype=np.int64)
    ref = oracle.taylor_attention(cat(pre.q, dec.q), cat(pre.k, dec.k), cat(pre.v, dec.v), wl.P, rows=rows)
    per_step = np.max(np.max(np.abs(got - ref), axis=-1) / np.max(np.abs(ref), axis=-1), axis=(0, 1))
    say("  err %.3e (first 16 steps %.3e, last 16 steps %.3e)" % (per_step.max(), per_step[:16].max(),
                                                                  per_step[-16:].max()))
    assert per_step.max() <= TOL_F32


def test_decode_d64_after_32768_token_prefix(sata, oracle):
    """Decode after a longer fp32 prefix (the 32768-token latency case): one
    sequence of 2 heads, sampled prefill rows and 16 decode steps against the
    oracle at the fp32 bar."""
    d, P, n, t = 64, 4, 32768, 16
    x = si.draw_qkv((1, 2), n + t, d, d, 32768 + 5, "f32")
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, 2)
    q, k, v = dev_all(x)
    say("decode after a %d-token prefix" % n)
    o = prefill(idx, st, q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous())
    od = [decode(idx, st, q[:, :, i].contiguous(), k[:, :, i].contiguous(), v[:, :, i].contiguous())
          for i in range(n, n + t)]
    rows = sample_rows(n, 128, 24, 3)
    ref = oracle.taylor_attention(x.q, x.k, x.v, P, rows=np.concatenate([rows, np.arange(n, n + t)]))
    err = rel_err(o.cpu().numpy()[:, :, rows], ref[:, :, :len(rows)])
    errd = rel_err(torch.stack(od, dim=2).cpu().numpy(), ref[:, :, len(rows):])
    say("  prefill err %.3e, decode err %.3e" % (err, errd))
    assert err <= TOL_F32 and errd <= TOL_F32
