"""The persistent prefill scan's error path, forced from the host: with the
fault-injection hook the scan skips its first work items, so their successors'
bounded waits for a predecessor's state run out.  Every kernel still ends
normally; the failure is recorded in the state's error word and reported as
SATA_ERR_HIP by sata_state_check and by the next call on the state, after
which the state works again."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import TOL_BF16, TOL_F32, dev_all, prefill, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as _sata
    _sata.load()
    return _sata


# Shapes with more work items than compute units, so each slice's chunks run as sub-segments
# (2 at d = 16 fp32 over 32 chunks; 4 at d = 32 bf16 over 256 chunks, the fp16-operand scan
# taking sub-segments of at least 64 chunks) whose items wait for their predecessors.
@pytest.mark.parametrize("d,dtype,chunk,nh,n", [(16, "f32", 128, 320, 4096), (32, "bf16", 64, 64, 16384)])
def test_timed_out_wait_is_reported(sata, oracle, d, dtype, chunk, nh, n):
    P = 4
    x = si.draw_qkv((1, nh), n, d, d, 5150 + d, dtype)
    idx = sata.Index(d, d, P)
    st = sata.State(idx, 1, nh)
    q, k, v = dev_all(x)
    plan = sata.sata_describe_prefill_plan(d, P, nh, n, chunk, sata.SATA_BF16 if dtype == "bf16" else sata.SATA_F32)
    say("scan error path: d=%d %s, %d heads x %d tokens, %d slices per head" % (d, dtype, nh, n, plan["slices"]))
    try:
        sata.sata_debug_scan_faults(item_base=3, spin_limit=256)
        prefill(idx, st, q, k, v, chunk=chunk)
        with pytest.raises(sata.SataError) as ei:
            sata.sata_state_check(st)
        assert ei.value.status == sata.SATA_ERR_HIP
        assert "gave up waiting" in str(ei.value)
        sata.sata_state_check(st)                       # reported once, then cleared
        # the next call on the state reports a failure recorded since the last report
        prefill(idx, st, q, k, v, chunk=chunk)
        torch.cuda.synchronize()
        with pytest.raises(sata.SataError) as ei:
            prefill(idx, st, q[:, :, :8].contiguous(), k[:, :, :8].contiguous(), v[:, :, :8].contiguous())
        assert ei.value.status == sata.SATA_ERR_HIP
    finally:
        sata.sata_debug_scan_faults(0, 0)
    # hook off: a fresh prefill on the same state is correct and reports nothing
    sata.sata_state_reset(st)
    o = prefill(idx, st, q, k, v, chunk=chunk)
    sata.sata_state_check(st)
    heads = [0, 1, 2, nh - 1]
    rows = np.array([0, 1, 127, 2048, n // 2 + 5, n - 1])
    sub = lambda a: np.ascontiguousarray(a[:, heads])
    ref = oracle.taylor_attention(sub(x.q), sub(x.k), sub(x.v), P, rows=rows)
    err = rel_err(o.float().cpu().numpy()[:, heads][:, :, rows], ref)
    say("  after the hook: err %.3e" % err)
    assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16)


def test_debug_hook_rejects_negative_arguments(sata):
    with pytest.raises(sata.SataError) as ei:
        sata.sata_debug_scan_faults(-1, 0)
    assert ei.value.status == sata.SATA_ERR_INVALID
    with pytest.raises(sata.SataError):
        sata.sata_debug_scan_faults(0, -5)
    sata.sata_debug_scan_faults(0, 0)
