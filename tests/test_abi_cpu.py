"""C-ABI and host logic, without a GPU: the library loads, exports every symbol
include/sata.h declares, validates arguments before touching a device, and its
host-built feature tables match the oracle's brute-force basis."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sata.h")


@pytest.fixture(scope="module")
def lib():
    from constant_cost_attention_amd import sata
    return sata.load()


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sata_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_symbols()
    for required in ("sata_build_index", "sata_state_alloc", "sata_prefill", "sata_decode_step"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    from constant_cost_attention_amd import sata
    names = _declared_symbols()
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(sata.exported_symbols()) == names


def test_status_strings(lib):
    from constant_cost_attention_amd import sata
    assert sata.status_string(0) == "ok"
    assert "invalid" in sata.status_string(1)
    assert "unsupported" in sata.status_string(2)
    assert "memory" in sata.status_string(3)
    assert "HIP" in sata.status_string(4)


def test_argument_checks_before_any_device_call(lib):
    from constant_cost_attention_amd import sata
    out = ctypes.c_void_p()
    assert lib.sata_build_index(64, 64, 4, None) == sata.SATA_ERR_INVALID
    assert lib.sata_build_index(0, 64, 4, ctypes.byref(out)) == sata.SATA_ERR_INVALID
    assert lib.sata_build_index(64, 64, 0, ctypes.byref(out)) == sata.SATA_ERR_INVALID
    assert lib.sata_build_index(12, 12, 4, ctypes.byref(out)) == sata.SATA_ERR_UNSUPPORTED
    assert lib.sata_build_index(64, 64, 6, ctypes.byref(out)) == sata.SATA_ERR_UNSUPPORTED
    assert b"P <=" in lib.sata_last_error()
    assert lib.sata_build_index(64, 128, 4, ctypes.byref(out)) == sata.SATA_ERR_UNSUPPORTED
    assert lib.sata_build_index(128, 64, 4, ctypes.byref(out)) == sata.SATA_ERR_UNSUPPORTED
    assert b"128" in lib.sata_last_error()
    assert lib.sata_index_features(None) == -1
    assert lib.sata_prefill(None, None, None, None, None, None, 16, 0, 0, 0, None) == sata.SATA_ERR_INVALID
    assert lib.sata_decode_step(None, None, None, None, None, None, 0, 0, None) == sata.SATA_ERR_INVALID
    assert lib.sata_state_alloc(None, 1, 1, None, ctypes.byref(out)) == sata.SATA_ERR_INVALID
    assert lib.sata_state_reset(None, None) == sata.SATA_ERR_INVALID
    assert lib.sata_expand_features(None, None, None, 1, 0, 0, None) == sata.SATA_ERR_INVALID
    assert lib.sata_prefill_backward(None, 1, 1, None, None, None, None, None, None, None, 8, 0, 0, 0,
                                     None) == sata.SATA_ERR_INVALID
    assert lib.sata_state_alloc_dtype(None, 1, 1, 1, None, ctypes.byref(out)) == sata.SATA_ERR_INVALID
    assert lib.sata_state_convert(None, None, None) == sata.SATA_ERR_INVALID
    assert lib.sata_state_set_decode_window(None, 4, None) == sata.SATA_ERR_INVALID
    assert lib.sata_state_flush(None, None) == sata.SATA_ERR_INVALID
    lib.sata_index_free(None)
    lib.sata_state_free(None)


@pytest.mark.parametrize("d,P", [(8, 1), (8, 3), (16, 4), (32, 4), (64, 4), (64, 2), (8, 5), (16, 5), (128, 3)])
def test_feature_tables_match_bruteforce_basis(oracle, d, P):
    """Host index builder vs oracle: same sorted tuples in the same order (orders
    0..P-1, lexicographic within an order), and readout weight
    1/(alpha! d^(p/2)) = count/(p! d^(p/2)) with count the brute-force group size."""
    from constant_cost_attention_amd import sata
    tup, coef = sata.sata_describe_features(d, P)
    assert len(tup) == oracle.cumulative_basis(d, P)
    f = 0
    for p in range(P):
        if d == 64 and p == 3:
            btup, bcnt = oracle.basis_bruteforce(d, p)
        else:
            btup, bcnt = oracle.basis_bruteforce(d, p)
        g = len(bcnt)
        t = tup[f:f + g]
        slots = np.stack([(t >> (8 * r)) & 0xFF for r in range(4)], axis=1).astype(np.int64)
        assert np.all(np.sum(slots < d, axis=1) == p)
        assert np.array_equal(slots[:, :p], btup.astype(np.int64))
        assert np.all(slots[:, p:] == d)
        expect = bcnt.astype(np.float64) / (math.factorial(p) * math.sqrt(d) ** p)
        np.testing.assert_allclose(coef[f:f + g].astype(np.float64), expect, rtol=1e-7, atol=0)
        f += g
    assert f == len(tup)


def test_describe_rejects_what_build_rejects(lib):
    from constant_cost_attention_amd import sata
    assert lib.sata_describe_features(12, 4, None, None, 0) == -1
    assert lib.sata_describe_features(64, 6, None, None, 0) == -1
    assert lib.sata_describe_features(64, 4, None, None, 0) == 47905
    assert lib.sata_describe_features(64, 5, None, None, 0) == 814385
    assert lib.sata_describe_features(128, 4, None, None, 0) == 366145
    assert lib.sata_describe_quads(128, 4, None, None, None, 0) == 0          # no prefill above d_K = 64


def test_binding_rejects_cpu_tensors():
    import torch
    from constant_cost_attention_amd import sata
    with pytest.raises(ValueError):
        sata._dev_ptr(torch.zeros(4), "q")


@pytest.mark.parametrize("d,P", [(8, 1), (8, 2), (8, 3), (16, 4), (32, 4), (64, 4), (8, 5), (16, 5), (32, 5)])
def test_quads_cover_every_feature_once(d, P):
    """Every valid quad slot is the feature (i0, i1, i2, 4b+z) at state index
    cidx + (z - first valid slot), with the feature table's readout weight;
    together the valid slots cover every feature exactly once except feature
    0, the constant order 0, which the prefill keeps out of the quads (P = 1
    has no quads at all); padding slots carry weight 0; the four quads of a
    position share the block b."""
    from constant_cost_attention_amd import sata
    tup, coef = sata.sata_describe_features(d, P)
    w0, cidx, qc = sata.sata_describe_quads(d, P)
    assert len(w0) % 4 == 0
    slots = np.stack([(tup >> (8 * r)) & 0xFF for r in range(4)], axis=1).astype(np.int64)
    order = np.sum(slots < d, axis=1).astype(np.int64)
    seen = np.zeros(len(tup), dtype=np.int64)
    for q in range(len(w0)):
        i1, i2, i0 = int(w0[q] & 0xFF), int((w0[q] >> 8) & 0xFF), int((w0[q] >> 16) & 0xFF)
        b, mask = int((w0[q] >> 24) & 0xF), int(w0[q] >> 28)
        assert b == int((w0[q - q % 4] >> 24) & 0xF)
        if not mask:
            assert cidx[q] == -1
            assert np.all(qc[q] == 0)
            continue
        z0 = (mask & -mask).bit_length() - 1
        for z in range(4):
            if not (mask >> z) & 1:
                assert qc[q, z] == 0
                continue
            f = int(cidx[q]) + z - z0
            idx = [i for i in (i0, i1, i2) if i < d]
            idx.append(4 * b + z)
            want = sorted(idx)
            assert idx == want
            assert [int(x) for x in slots[f, :order[f]]] == want, (q, z, want)
            # quad weight = multinomial part; the feature weight also carries d^(-p/2)
            assert abs(qc[q, z] / math.sqrt(d) ** len(want) - coef[f]) <= 1e-6 * coef[f]
            seen[f] += 1
    assert seen[0] == 0 and order[0] == 0
    assert np.all(seen[1:] == 1)


def _positions16(d, P):
    """Positions of the 16-stream view by its construction rule, counted without the library:
    per block a the prefixes whose last index lies in it (order 3: i1 <= i2, order 2: i2
    alone, and the empty prefix for a = 0); groups of 16 per block for P = 4, pooled over
    the whole list for P <= 3; a group sweeps the blocks from its first prefix's to the last."""
    per = []
    for a in range(d // 4):
        n = (1 if P >= 2 and a == 0 else 0) + (4 if P >= 3 else 0)
        if P >= 4:
            n += sum(i2 + 1 for i2 in range(4 * a, 4 * a + 4))
        per.append(n)
    if P <= 3:
        blocks = [a for a in range(d // 4) for _ in range(per[a])]
        return sum(d // 4 - blocks[g] for g in range(0, len(blocks), 16))
    return sum(-(-per[a] // 16) * (d // 4 - a) for a in range(d // 4))


@pytest.mark.parametrize("d,P", [(16, 2), (16, 3), (16, 4), (32, 3), (64, 3), (64, 4), (128, 3), (128, 4)])
def test_quads16_cover_every_feature_once(d, P):
    """The fp16-operand scan's view: every valid slot is the feature (i1, i2, 4b+z) at state
    index cidx + (z - first valid slot) with the feature table's weight, and the valid slots
    cover every feature but the constant one exactly once.  The 16 quads of a position share
    the block b; flag bit 1 marks exactly the positions whose 16 prefixes differ from the
    previous position's, and within a group b steps by one; a position without flag bit 0
    has only full quads of one weight (and padding).  The position count follows the
    grouping rule (P <= 3 pools the prefixes of all blocks: 44 positions at d = 64, against
    136 with groups per block)."""
    from constant_cost_attention_amd import sata
    tup, coef = sata.sata_describe_features(d, P)
    w0, cidx, qc, flags = sata.sata_describe_quads16(d, P)
    assert len(w0) == _positions16(d, P)
    if (d, P) == (64, 3):
        assert len(w0) == 44
    slots = np.stack([(tup >> (8 * r)) & 0xFF for r in range(4)], axis=1).astype(np.int64)
    order = np.sum(slots < d, axis=1).astype(np.int64)
    seen = np.zeros(len(tup), dtype=np.int64)
    prev_pref, prev_b = None, None
    for p in range(len(w0)):
        i1 = (w0[p] & 0xFF).astype(np.int64)
        i2 = ((w0[p] >> 8) & 0xFF).astype(np.int64)
        b = ((w0[p] >> 16) & 0xFF).astype(np.int64)
        mask = (w0[p] >> 28).astype(np.int64)
        assert np.all(b == b[0])
        pref = (tuple(i1), tuple(i2))
        starts = prev_pref is None or pref != prev_pref
        assert bool(flags[p] & 2) == starts, p
        if not starts:
            assert b[0] == prev_b + 1
        prev_pref, prev_b = pref, int(b[0])
        pad = (i1 == d + 1) & (i2 == d + 1)
        mixed = False
        for s in range(16):
            if pad[s]:
                assert mask[s] == 0 and cidx[p, s] == -1 and np.all(qc[p, s] == 0)
                continue
            if mask[s] != 0xF or len(set(qc[p, s].tolist())) != 1:
                mixed = True
            if not mask[s]:
                assert cidx[p, s] == -1 and np.all(qc[p, s] == 0)
                continue
            z0 = (int(mask[s]) & -int(mask[s])).bit_length() - 1
            for z in range(4):
                if not (mask[s] >> z) & 1:
                    assert qc[p, s, z] == 0
                    continue
                f = int(cidx[p, s]) + z - z0
                idx = [int(i) for i in (i1[s], i2[s]) if i < d] + [4 * int(b[0]) + z]
                assert idx == sorted(idx)
                assert [int(x) for x in slots[f, :order[f]]] == idx, (p, s, z, idx)
                assert abs(qc[p, s, z] / math.sqrt(d) ** len(idx) - coef[f]) <= 1e-6 * coef[f]
                seen[f] += 1
        assert bool(flags[p] & 1) == mixed, p
    assert seen[0] == 0 and order[0] == 0
    assert np.all(seen[1:] == 1)
    assert sata.sata_describe_quads16(8, 4)[0].shape == (0, 16)



def test_describe_errors_raise_sata_error():
    """The binding's describe calls turn a rejected (d_k, P) into SataError with the
    library's status and message (an unsupported head size is SATA_ERR_UNSUPPORTED)."""
    from constant_cost_attention_amd import sata
    with pytest.raises(sata.SataError) as ei:
        sata.sata_describe_features(12, 4)
    assert ei.value.status == sata.SATA_ERR_UNSUPPORTED
    assert "head dims" in str(ei.value)
    with pytest.raises(sata.SataError) as ei:
        sata.sata_describe_quads(64, 6)
    assert ei.value.status == sata.SATA_ERR_UNSUPPORTED
    with pytest.raises(sata.SataError) as ei:
        sata.sata_describe_features(0, 4)
    assert ei.value.status == sata.SATA_ERR_INVALID


def test_prefill_plan_shrinks_segments_under_a_smaller_cap():
    """Workspace re-planning: under a smaller cap the plan keeps the same slices, takes fewer
    chunks per segment, and its workspace fits the cap (down to one chunk per segment, which
    may exceed it); the default cap runs the headline workload (1 x 8 x 65536, d = 64, bf16)
    as one segment."""
    from constant_cost_attention_amd import sata
    full = sata.sata_describe_prefill_plan(64, 4, 8, 65536, 128, sata.SATA_BF16)
    assert full["seg_chunks"] == 512
    caps = [full["work_bytes"] // 2, full["work_bytes"] // 7, 1 << 26, 1]
    prev = full
    for cap in caps:
        p = sata.sata_describe_prefill_plan(64, 4, 8, 65536, 128, sata.SATA_BF16, work_cap=cap)
        assert p["slices"] == full["slices"]
        assert 1 <= p["seg_chunks"] <= prev["seg_chunks"]
        assert p["work_bytes"] <= cap or p["seg_chunks"] == 1
        prev = p
    assert prev["seg_chunks"] == 1
    # halving the failed workspace (what sata_prefill does on SATA_ERR_OOM) always makes progress
    cap, segs = 16 << 30, []
    while True:
        p = sata.sata_describe_prefill_plan(16, 4, 64, 131072, 128, sata.SATA_BF16, work_cap=cap)
        segs.append(p["seg_chunks"])
        if p["seg_chunks"] == 1:
            break
        cap = p["work_bytes"] // 2
    assert all(a > b for a, b in zip(segs, segs[1:]))
    # head size 128: chunked only on the fp16-operand scan (bf16 inputs, P <= 4)
    for bad in ((128, 4, sata.SATA_F32), (128, 5, sata.SATA_BF16)):
        with pytest.raises(sata.SataError):
            sata.sata_describe_prefill_plan(bad[0], bad[1], 8, 4096, 0, bad[2])


def test_prefill_plan_head_size_128():
    """d_K = 128 (bf16, P <= 4): one position per update wavefront, so a slice holds 4 x 64
    features; 64-token chunks whatever the request; the 1 x 8 x 4096 workload in one segment."""
    from constant_cost_attention_amd import sata
    P = 4
    feats = sum(math.comb(128 + p - 1, p) for p in range(1, P))   # orders 1 .. P-1 (order 0 is outside)
    p64 = sata.sata_describe_prefill_plan(128, P, 8, 4096, 0, sata.SATA_BF16)
    assert p64 == sata.sata_describe_prefill_plan(128, P, 8, 4096, 128, sata.SATA_BF16)
    assert p64["slices"] >= feats / 256
    assert p64["seg_chunks"] == 4096 // 64
    # partials (fp16) of every slice of every chunk fit the default workspace
    assert 8 * p64["slices"] * 4096 * 129 * 2 <= p64["work_bytes"] <= 16 << 30


def test_forced_positions_change_the_plan():
    """sata_debug_prefill_positions: one position per update wavefront at d_K = 64
    doubles the slices of the rule's two; values other than 0, 1, 2, 3, 5 are
    refused; 0 restores the rule."""
    from constant_cost_attention_amd import sata
    rule = sata.sata_describe_prefill_plan(64, 4, 8, 65536, 128, sata.SATA_BF16)["slices"]
    try:
        sata.sata_debug_prefill_positions(1)
        one = sata.sata_describe_prefill_plan(64, 4, 8, 65536, 128, sata.SATA_BF16)["slices"]
        sata.sata_debug_prefill_positions(5)   # not held at d_K = 64: the rule applies
        five = sata.sata_describe_prefill_plan(64, 4, 8, 65536, 128, sata.SATA_BF16)["slices"]
        for bad in (-1, 4, 6):
            with pytest.raises(sata.SataError):
                sata.sata_debug_prefill_positions(bad)
    finally:
        sata.sata_debug_prefill_positions(0)
    assert one in (2 * rule - 1, 2 * rule) and five == rule
    assert sata.sata_describe_prefill_plan(64, 4, 8, 65536, 128, sata.SATA_BF16)["slices"] == rule


def test_forced_refresh_interval_checks():
    """sata_debug_prefill_refresh takes 0 (the rule) or 1 .. 16 chunks and refuses
    anything else with SATA_ERR_INVALID; it does not change the plan's slices or
    workspace (the interval only moves terms between the scan and the reduce)."""
    from constant_cost_attention_amd import sata
    rule = sata.sata_describe_prefill_plan(64, 4, 8, 65536, 128, sata.SATA_BF16)
    try:
        for ok in (1, 3, 16):
            sata.sata_debug_prefill_refresh(ok)
            assert sata.sata_describe_prefill_plan(64, 4, 8, 65536, 128, sata.SATA_BF16) == rule
        for bad in (-1, 17, 1000):
            with pytest.raises(sata.SataError) as e:
                sata.sata_debug_prefill_refresh(bad)
            assert e.value.status == sata.SATA_ERR_INVALID
    finally:
        sata.sata_debug_prefill_refresh(0)
