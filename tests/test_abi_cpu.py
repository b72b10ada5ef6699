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
    return sorted(set(re.findall(r"\b(sata_[a-z_]+)\s*\(", text)))


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
