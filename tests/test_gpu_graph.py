"""Decode steps captured in a HIP graph (torch.cuda.graph drives the capture
on its own stream; the library only launches kernels there, allocates nothing
after a state's first step and records no memset nodes) and replayed with new
tokens copied into the captured input buffers, against the same steps run
eagerly.  A windowed decode is captured a whole window at a time: which
steps read and which one folds is decided on the host at capture."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import TOL_BF16, TOL_F32, decode, dev_all, prefill, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as s
    s.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return s


@pytest.mark.parametrize("window", [1, 4])
def test_decode_steps_replayed_from_a_graph(sata, oracle, window):
    d, P, heads, n0 = 16, 4, 4, 100
    reps = 5                                   # graph replays
    T = window * (reps + 1)                    # one eager window first (allocates), then the replays
    x = si.draw_qkv((1, heads), n0 + T, d, d, 5000 + window, "f32")
    idx = sata.Index(d, d, P)
    q, k, v = dev_all(x)
    say("decode in a HIP graph, window %d, %d replays" % (window, reps))
    st = sata.State(idx, 1, heads)
    prefill(idx, st, q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous())
    sata.sata_state_set_decode_window(st, window)
    tok = lambda a, t: a[:, :, t].contiguous()
    outs = [decode(idx, st, tok(q, t), tok(k, t), tok(v, t)) for t in range(n0, n0 + window)]
    torch.cuda.synchronize()
    # static buffers: one slot per step of the window
    sq = [torch.empty((1, heads, d), device="cuda") for _ in range(window)]
    sk = [torch.empty_like(sq[0]) for _ in range(window)]
    sv = [torch.empty_like(sq[0]) for _ in range(window)]
    so = [torch.empty_like(sq[0]) for _ in range(window)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for w in range(window):
            sata.sata_decode_step(idx, st, sq[w], sk[w], sv[w], so[w])
    for r in range(reps):
        t0 = n0 + window * (r + 1)
        for w in range(window):
            sq[w].copy_(tok(q, t0 + w)); sk[w].copy_(tok(k, t0 + w)); sv[w].copy_(tok(v, t0 + w))
        graph.replay()
        torch.cuda.synchronize()                 # eager work and a sync between replays
        outs.extend(o.clone() for o in so)
    o = torch.stack(outs, dim=2).cpu().numpy()
    ref = oracle.taylor_attention(x.q, x.k, x.v, P, rows=np.arange(n0, n0 + T, dtype=np.int64))
    err = rel_err(o, ref)
    say("  err %.3e" % err)
    assert err <= TOL_F32


@pytest.mark.parametrize("d,heads,n", [(32, 3, 200), (64, 2, 300)])
def test_prefill_replayed_from_a_graph(sata, oracle, d, heads, n):
    """A state reset and a bf16 prefill captured once (after an eager call of
    the same size, which sizes the workspace) and replayed on new inputs
    copied into the captured buffers: every replay against the oracle."""
    P, reps = 4, 3
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, heads)
    draws = [si.draw_qkv((1, heads), n, d, d, 7100 + 10 * d + r, "bf16") for r in range(reps + 1)]
    say("prefill in a HIP graph, d=%d heads=%d n=%d, %d replays" % (d, heads, n, reps))
    sq, sk, sv = dev_all(draws[0])
    so = torch.empty(sv.shape, dtype=torch.float32, device="cuda")
    sata.sata_prefill(idx, st, sq, sk, sv, so)                 # eager: sizes the workspace
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sata.sata_state_reset(st)
        sata.sata_prefill(idx, st, sq, sk, sv, so)
    for r in range(1, reps + 1):
        q, k, v = dev_all(draws[r])
        sq.copy_(q); sk.copy_(k); sv.copy_(v)
        graph.replay()
        torch.cuda.synchronize()
        err = rel_err(so.cpu().numpy(), oracle.taylor_attention(draws[r].q, draws[r].k, draws[r].v, P))
        say("  replay %d: err %.3e" % (r, err))
        assert err <= TOL_BF16
    st.free()
    idx.free()
