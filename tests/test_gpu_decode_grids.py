"""The decode step and the read kernel of a deferred decode have two grids:
with few heads each feature tile's d_V + 1 state rows are split over
workgroups; with many, a workgroup takes all rows of a tile (the plain step)
or several tiles (the read kernel).  The same heads are decoded both ways
(alone, and as the first heads of a batch large enough for the whole-tile
grid) and must agree to fp32 rounding; sampled heads of both runs against the
oracle (O1, or O8 for a bf16-stored state)."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from sata_testutil import TOL_F32, decode, dev_all, prefill, rel_err, say

pytestmark = pytest.mark.gpu

TOL_BF16_STATE = 1e-3
DRIFT_SHARE = 1e-2


@pytest.fixture(scope="module")
def sata():
    from constant_cost_attention_amd import sata as s
    s.load()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return s


def _run(sata, idx, heads, x, n0, T, window, dtype):
    """prefill n0 tokens into an fp32 state (converted to bf16 if asked), then
    T decode steps at the given window; outputs [1, heads, T, d_V]."""
    sl = lambda a: a[:, :heads].contiguous()
    q, k, v = (sl(t) for t in dev_all(x))
    st = sata.State(idx, 1, heads)
    prefill(idx, st, q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(), v[:, :, :n0].contiguous())
    if dtype == "bf16":
        st16 = sata.State(idx, 1, heads, dtype=torch.bfloat16)
        sata.sata_state_convert(st, st16)
        st.free()
        st = st16
    sata.sata_state_set_decode_window(st, window)
    outs = [decode(idx, st, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous())
            for t in range(n0, n0 + T)]
    st.free()
    return torch.stack(outs, dim=2).cpu().numpy()


# (d, P, heads of the whole-tile run, state dtype): heads x feature tiles of
# 1024 (fp32) or 2048 (bf16) features reach 8192 workgroups
@pytest.mark.parametrize("d,P,big,dtype", [(64, 4, 176, "f32"), (32, 4, 1176, "f32"), (16, 4, 8192, "f32"),
                                           (8, 4, 8192, "f32"), (64, 4, 344, "bf16"), (64, 3, 2736, "f32")])
@pytest.mark.parametrize("window", [1, 4])
def test_split_and_whole_tile_grids_agree(sata, oracle, d, P, big, dtype, window):
    small, n0, T = 6, 20, 6
    x = si.draw_qkv((1, big), n0 + T, d, d, 6100 + d + P, "f32")
    idx = sata.Index(d, d, P)
    say("decode grids d=%d P=%d %s state, window %d: %d heads vs %d" % (d, P, dtype, window, small, big))
    a = _run(sata, idx, small, x, n0, T, window, dtype)
    b = _run(sata, idx, big, x, n0, T, window, dtype)
    diff = rel_err(a, b[:, :small])
    say("  split vs whole-tile %.3e" % diff)
    assert diff <= (TOL_F32 if dtype == "f32" else TOL_BF16_STATE)
    for h in (0, big - 1):
        sub = lambda t: t[:, h:h + 1]
        rows = np.arange(n0, n0 + T, dtype=np.int64)
        exact = oracle.taylor_attention(sub(x.q), sub(x.k), sub(x.v), P, rows=rows)
        got = b[:, h:h + 1]
        if dtype == "f32":
            err = rel_err(got, exact)
            say("  head %d vs O1 %.3e" % (h, err))
            assert err <= TOL_F32
        else:
            ref = oracle.bf16_state_decode(sub(x.q), sub(x.k), sub(x.v), P, n0, window=window)
            err, drift = rel_err(got, ref), rel_err(ref, exact)
            say("  head %d vs O8 %.3e (drift %.3e)" % (h, err, drift))
            assert err <= TOL_BF16_STATE + DRIFT_SHARE * drift
