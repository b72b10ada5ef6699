"""The allocation-free prefill (sata_prefill_noalloc, called through the C ABI by the
binding) against sata_prefill on the same seeded inputs: outputs and final states
agree, for two calls in a row of which the second is smaller (fresh states, and the
first state continued), so nothing left in the shared scratch array by one call
reaches the next.  Covered: the fp16-operand scan (bf16 inputs, d = 32 and a d = 64
call that the scratch splits into one-chunk segments while sata_prefill runs it in
one), the general scan (fp32 inputs, d = 8), and the refusal of a call whose
single-chunk segments need more workspace than the scratch holds."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import TOL_BF16, TOL_F32, dev_all, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as _sata
    _sata.load()
    return _sata


def _run(sata, fn, idx, st, q, k, v):
    out = torch.empty(v.shape, dtype=torch.float32, device=v.device)
    fn(idx, st, q, k, v, out)
    return out


def _state_err(a, b) -> float:
    a = a.double().cpu().numpy().ravel()
    b = b.double().cpu().numpy().ravel()
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# (d, P, dtype, heads, n of the first call, n of the second call)
CASES = [
    (32, 4, "bf16", 6, 700, 200),     # fp16-operand scan, ragged last chunk
    (8, 3, "f32", 5, 300, 65),        # general scan (fp32 inputs)
    (64, 4, "bf16", 72, 384, 130),    # 72 heads: one-chunk segments in the scratch
]


@pytest.mark.parametrize("d,P,dtype,nh,n1,n2", CASES)
def test_noalloc_matches_prefill(sata, d, P, dtype, nh, n1, n2):
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    idx = sata.Index(d, d, P)
    try:
        for call, n in enumerate((n1, n2)):
            say("no-alloc prefill: d=%d P=%d %s, %d heads x %d tokens (call %d)" % (d, P, dtype, nh, n, call + 1))
            x = si.draw_qkv((1, nh), n, d, d, 7100 + 10 * d + call, dtype)
            q, k, v = dev_all(x)
            a, b = sata.State(idx, 1, nh), sata.State(idx, 1, nh)
            oa = _run(sata, sata.sata_prefill_noalloc, idx, a, q, k, v)
            ob = _run(sata, sata.sata_prefill, idx, b, q, k, v)
            torch.cuda.synchronize()
            sata.sata_state_check(a)
            err_o = rel_err(oa.cpu().numpy(), ob.cpu().numpy())
            err_s = _state_err(sata.state_tensor(a), sata.state_tensor(b))
            say("  out err %.3e, state err %.3e, identical %s" % (err_o, err_s, bool(torch.equal(oa, ob))))
            assert np.isfinite(oa.cpu().numpy()).all()
            assert err_o <= tol and err_s <= tol
            a.free()
            b.free()
            del q, k, v, oa, ob
            torch.cuda.empty_cache()
    finally:
        idx.free()


def test_noalloc_continues_a_state(sata):
    """A second, smaller call on the state of the first continues the sequence as sata_prefill does."""
    d, P, nh = 32, 4, 4
    idx = sata.Index(d, d, P)
    x = si.draw_qkv((1, nh), 600, d, d, 7300, "bf16")
    q, k, v = dev_all(x)
    a, b = sata.State(idx, 1, nh), sata.State(idx, 1, nh)
    say("no-alloc prefill continued: d=32 P=4 bf16, 4 heads, 450 + 150 tokens")
    parts = [(0, 450), (450, 600)]
    for lo, hi in parts:
        sl = lambda t: t[:, :, lo:hi].contiguous()
        oa = _run(sata, sata.sata_prefill_noalloc, idx, a, sl(q), sl(k), sl(v))
        ob = _run(sata, sata.sata_prefill, idx, b, sl(q), sl(k), sl(v))
        torch.cuda.synchronize()
        err = rel_err(oa.cpu().numpy(), ob.cpu().numpy())
        say("  tokens %d..%d: out err %.3e" % (lo, hi, err))
        assert err <= TOL_BF16
    assert _state_err(sata.state_tensor(a), sata.state_tensor(b)) <= TOL_BF16
    a.free()
    b.free()
    idx.free()


def test_noalloc_refuses_oversized_workspace(sata):
    """96 heads of d = 64, P = 4 need about 1.6 MB of workspace per head even in one-chunk
    segments, more than the 128 MiB scratch: refused before any launch, state untouched."""
    d, P, nh, n = 64, 4, 96, 128
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, nh)
    say("no-alloc prefill refusal: d=64 P=4 bf16, 96 heads x 128 tokens")
    q = torch.zeros((1, nh, n, d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((1, nh, n, d), dtype=torch.float32, device="cuda")
    with pytest.raises(sata.SataError) as ei:
        sata.sata_prefill_noalloc(idx, st, q, q, q, out)
    assert ei.value.status == sata.SATA_ERR_UNSUPPORTED
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert float(sata.state_tensor(st).abs().max()) == 0.0
    st.free()
    idx.free()
