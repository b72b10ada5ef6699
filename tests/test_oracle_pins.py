"""Pins of the oracle against what the pages and mathematics fix (CPU only).

Each test names the plausible oracle mistake it would catch.  The pages print
no worked SATA output, so exact outputs are pinned by closed forms, special
cases that reduce to textbook/library routines, exact rational arithmetic on
tiny inputs, and invariants.
"""
import collections
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _rand_qkv(seed, lead, n, dk, dv):
    d = si.draw_qkv(lead, n, dk, dv, seed, "f32")
    return d.q, d.k, d.v


# ------------------------------------------------------------ basis (O3, O4)

@pytest.mark.parametrize("d", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("p", [0, 1, 2, 3, 4])
def test_basis_count_is_binomial(oracle, d, p):
    """Brute-force sorted-tuple groups of all d^p ordered tuples number
    C(d+p-1, p) [hotdry, 'Core insight of symmetric tensor decomposition'].
    Catches a wrong grouping (e.g. keeping ordered tuples, or strict i1<i2)."""
    tup, cnt = oracle.basis_bruteforce(d, p)
    assert len(cnt) == math.comb(d + p - 1, p)
    assert int(cnt.sum()) == d ** p
    # every group is a sorted tuple, listed in lexicographic order
    for t in tup:
        assert list(t) == sorted(t)
    assert [tuple(t) for t in tup] == sorted(tuple(t) for t in tup)


@pytest.mark.parametrize("d,p", [(3, 3), (4, 4), (5, 2), (2, 4)])
def test_group_sizes_are_multinomial(oracle, d, p):
    """Group size = p!/prod(alpha!) (textbook multinomial).  Catches a wrong
    symmetric weight in phi."""
    tup, cnt = oracle.basis_bruteforce(d, p)
    for t, c in zip(tup, cnt):
        mult = collections.Counter(t.tolist())
        expect = math.factorial(p)
        for a in mult.values():
            expect //= math.factorial(a)
        assert c == expect


def test_page_figures_minimal_basis_and_expansion(oracle):
    """The page's numbers: 47905 minimal-basis features at d_K=64 (read as the
    orders 0..3 together) and more than 16 million unreduced monomials at
    d_K=64, p=4 [hotdry, 'Core insight of symmetric tensor decomposition']."""
    g = json.load(open(GOLDEN))
    fig = g["minimal_basis_d64"]
    total = sum(len(oracle.basis_bruteforce(fig["d_k"], p)[1]) for p in range(fig["P"]))
    assert total == fig["page_value"] == oracle.cumulative_basis(64, 4)
    full = g["full_expansion_d64_p4"]
    _, cnt4 = oracle.basis_bruteforce(full["d_k"], full["p"])
    assert int(cnt4.sum()) > full["lower_bound"]
    # the single order p=4 alone is C(67,4), not the page's 47905
    assert len(cnt4) == math.comb(67, 4) == 766480


@pytest.mark.parametrize("d,P,expect", [(8, 3, 45), (16, 4, 969), (32, 4, 6545), (64, 4, 47905)])
def test_cumulative_basis_at_workloads(oracle, d, P, expect):
    total = sum(len(oracle.basis_bruteforce(d, p)[1]) for p in range(P))
    assert total == expect == oracle.cumulative_basis(d, P)


@pytest.mark.parametrize("seed", range(6))
def test_phi_identity_exact_on_integers(oracle, seed):
    """sum_t count_t prod q prod k = (q.k)^p exactly for integer q, k (both sides
    are exact integers in fp64), and phi_p(q).phi_p(k) = (q.k)^p to rounding.
    Catches a wrong index or weight in the feature map."""
    rng = np.random.default_rng(seed)
    for d in range(1, 5):
        for p in range(0, 5):
            q = rng.integers(-3, 4, size=d).astype(np.float64)
            k = rng.integers(-3, 4, size=d).astype(np.float64)
            tup, cnt = oracle.basis_bruteforce(d, p)
            lhs = 0.0
            for t, c in zip(tup, cnt):
                lhs += float(c) * float(np.prod(q[t])) * float(np.prod(k[t]))
            assert lhs == float(np.dot(q, k)) ** p
            sym = float(np.dot(oracle.phi(q, p), oracle.phi(k, p)))
            ref = float(np.dot(q, k)) ** p
            assert abs(sym - ref) <= 1e-12 * max(1.0, abs(ref))


# ------------------------------------------------------------ state form (O5)

@pytest.mark.parametrize("d,P", [(1, 1), (1, 4), (2, 2), (2, 3), (3, 4), (4, 4), (4, 3), (3, 1)])
def test_recurrent_state_equals_quadratic(oracle, d, P):
    """The constant-size state form (O5) equals the quadratic definition (O1)
    [hotdry, 'Engineering realisation of the constant compute cost'].
    Catches a missing 1/p!, a wrong d^(p/2), or a read-before-update."""
    q, k, v = _rand_qkv(100 + 10 * d + P, (2,), 40, d, 3)
    a = oracle.recurrent_attention(q, k, v, P)
    b = oracle.taylor_attention(q, k, v, P)
    assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))


def _fp32_floor_bound(q, k, v, P, o):
    """First-order bound on |O7 - O5| per output element.  With u = 2^-24 and
    gamma_N = N u / (1 - N u): every state element is a sum over the n tokens of
    products carrying at most P + 2 roundings each, and the readout sums the m
    features of an order, so each numerator or normaliser sum is exact up to
    gamma_N times the same sum taken over absolute values, N = n + m + 2P + 8.
    The absolute-value sum of the symmetric features is sum_p (|q|.|k|/sqrt d)^p/p!
    (the multinomial counts add up to the plain power), so
      |dy_c| <= gamma_N * sum_j wabs_j |v_jc|,  |dz| <= gamma_N * sum_j wabs_j,
    and o_c = y_c / z changes by at most (|dy_c| + |o_c| |dz|)/z + 2u|o_c|."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    n, d = q.shape[-2:]
    m = math.comb(d + P - 1, P - 1)
    u = 2.0 ** -24
    N = n + m + 2 * P + 8
    gam = N * u / (1 - N * u)
    x = np.einsum("...id,...jd->...ij", q, k) / math.sqrt(d)
    xa = np.einsum("...id,...jd->...ij", np.abs(q), np.abs(k)) / math.sqrt(d)
    w = sum(x ** p / math.factorial(p) for p in range(P))
    wa = sum(xa ** p / math.factorial(p) for p in range(P))
    causal = np.tril(np.ones((n, n)))
    w, wa = w * causal, wa * causal
    z = w.sum(-1)[..., None]
    dy = gam * (wa @ np.abs(v))
    dz = gam * wa.sum(-1)[..., None]
    return (dy + np.abs(o) * dz) / np.abs(z) + 2 * u * np.abs(o)


@pytest.mark.parametrize("d,P,n", [(4, 3, 300), (6, 4, 200), (8, 2, 400)])
def test_fp32_emulation_is_fp32(oracle, d, P, n):
    """O7 carries the recurrent form's sums in float: it stays within the
    first-order fp32 error bound of the exact form O5 everywhere (a dropped or
    wrong term would leave it), and it is measurably not fp64 (a version that
    kept double would sit within 1e-13 of O5)."""
    q, k, v = _rand_qkv(7 + d, (2,), n, d, d)
    a = oracle.recurrent_attention_f32(q, k, v, P)
    b = oracle.recurrent_attention(q, k, v, P)
    bound = _fp32_floor_bound(q, k, v, P, b)
    assert np.all(np.abs(a - b) <= bound)
    rel = np.max(np.abs(a - b)) / np.max(np.abs(b))
    assert rel > 1e-9, rel


def test_fp32_emulation_is_exact_on_dyadic_inputs(oracle):
    """On inputs whose every product and partial sum fits a float exactly
    (small dyadic rationals, few tokens), O7 equals O5 up to the final division
    rounding: the emulation rounds only where fp32 itself must."""
    rng = np.random.default_rng(17)
    d, P, n = 3, 3, 12
    q = (rng.integers(-4, 5, size=(1, n, d)) / 4.0).astype(np.float32)
    k = (rng.integers(-4, 5, size=(1, n, d)) / 4.0).astype(np.float32)
    v = (rng.integers(-8, 9, size=(1, n, d)) / 8.0).astype(np.float32)
    a = oracle.recurrent_attention_f32(q, k, v, P)
    b = oracle.recurrent_attention(q, k, v, P)
    # sqrt(count) and 1/(p! d^(p/2)) weights are irrational here, so equality is to fp32 rounding of
    # a handful of operations, far below the sums' floor on random inputs
    assert np.max(np.abs(a - b)) <= 64 * 2.0 ** -24 * np.max(np.abs(b))


# ------------------------------------------------------------ special cases (O1)

def test_P1_is_causal_running_mean(oracle):
    """P=1 keeps only the constant order: w = 1, so o_i is the mean of v_0..v_i.
    Catches j<i (diagonal dropped) or j<=n (non-causal)."""
    q, k, v = _rand_qkv(11, (3,), 50, 5, 6)
    o = oracle.taylor_attention(q, k, v, 1)
    vv = v.astype(np.float64)
    ref = np.cumsum(vv, axis=1) / np.arange(1, 51)[None, :, None]
    assert np.max(np.abs(o - ref)) < 1e-13


def _torch_softmax_attention(q, k, v):
    """Causal scaled-dot-product softmax attention via torch library routines
    (CPU, float64) [mokono, standard attention]."""
    qt, kt, vt = (torch.from_numpy(np.asarray(x, dtype=np.float64)) for x in (q, k, v))
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) / math.sqrt(q.shape[-1])
    n = q.shape[-2]
    mask = torch.ones(n, n, dtype=torch.bool).triu(1)
    s = s.masked_fill(mask, float("-inf"))
    return torch.matmul(torch.softmax(s, dim=-1), vt).numpy()


def test_softmax_oracle_matches_torch(oracle):
    q, k, v = _rand_qkv(12, (2, 2), 70, 8, 5)
    a = oracle.softmax_attention(q, k, v)
    b = _torch_softmax_attention(q, k, v)
    assert np.max(np.abs(a - b)) < 1e-12


def test_large_P_converges_to_softmax_library(oracle):
    """With P=24 orders the truncation error of exp on |x|<=1 is below
    e/24! ~ 4e-24 per weight, so the Taylor oracle must equal library softmax
    attention to rounding.  Catches a wrong 1/p!, a sign error in x, a missing
    1/sqrt(d) scale or a q/k swap."""
    q, k, v = _rand_qkv(13, (2, 3), 90, 16, 7)
    a = oracle.taylor_attention(q, k, v, 24)
    b = _torch_softmax_attention(q, k, v)
    assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("P", [3, 4])
def test_softmax_gap_below_truncation_bound(oracle, P):
    """|o_taylor - o_softmax| <= 2 eps/(1-eps) * max_j |v_j - o_softmax| with
    eps = max_{|x|<=1} |w_P(x) e^-x - 1| (Lagrange remainder; x in [-1,1] by
    the input recipe).  The gap the page compares with fp16 precision
    [hotdry, 'Precision/efficiency trade-off']."""
    xs = np.linspace(-1, 1, 20001)
    w = sum(xs ** p / math.factorial(p) for p in range(P))
    eps = float(np.max(np.abs(w * np.exp(-xs) - 1)))
    q, k, v = _rand_qkv(14, (2,), 200, 8, 4)
    a = oracle.taylor_attention(q, k, v, P)
    b = oracle.softmax_attention(q, k, v)
    vv = v.astype(np.float64)
    for h in range(2):
        for i in range(200):
            spread = np.max(np.abs(vv[h, : i + 1] - b[h, i][None, :]))
            assert np.max(np.abs(a[h, i] - b[h, i])) <= 2 * eps / (1 - eps) * spread + 1e-13


def test_single_token_returns_v0(oracle):
    q, k, v = _rand_qkv(15, (4,), 1, 6, 3)
    o = oracle.taylor_attention(q, k, v, 4)
    assert np.max(np.abs(o - v.astype(np.float64))) <= 4e-16 * np.max(np.abs(v))


def test_constant_v_gives_constant_output(oracle):
    q, k, _ = _rand_qkv(16, (2,), 64, 8, 3)
    v = np.tile(np.array([1.5, -2.25, 0.125], dtype=np.float32), (2, 64, 1))
    o = oracle.taylor_attention(q, k, v, 4)
    assert np.max(np.abs(o - v.astype(np.float64))) < 1e-13


def test_affine_equivariance_in_v(oracle):
    """v -> a v + b maps o -> a o + b (weights sum to one after normalising).
    Catches a missing or wrong normaliser."""
    q, k, v = _rand_qkv(17, (2,), 64, 8, 4)
    v = (np.round(v * 64) / 64).astype(np.float32)    # dyadic grid: a*v+b stays exact
    o = oracle.taylor_attention(q, k, v, 3)
    a, b = np.float32(2.0), np.float32(0.5)            # exact in fp32 for these v
    o2 = oracle.taylor_attention(q, k, v * a + b, 3)
    ref = o * 2.0 + 0.5
    assert np.max(np.abs(o2 - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_joint_coordinate_permutation_invariance(oracle):
    q, k, v = _rand_qkv(18, (2,), 64, 8, 4)
    perm = np.random.default_rng(0).permutation(8)
    o = oracle.taylor_attention(q, k, v, 4)
    o2 = oracle.taylor_attention(q[..., perm], k[..., perm], v, 4)
    assert np.max(np.abs(o - o2)) < 1e-13


def test_row_subset_matches_full(oracle):
    q, k, v = _rand_qkv(19, (3,), 100, 8, 4)
    rows = np.array([0, 5, 99, 42], dtype=np.int64)
    full = oracle.taylor_attention(q, k, v, 4)
    sub = oracle.taylor_attention(q, k, v, 4, rows=rows)
    assert np.array_equal(full[:, rows], sub)


def test_exact_rational_tiny_case(oracle):
    """Brute force in exact rational arithmetic on a tiny case with d_K=4, so
    that 1/sqrt(d_K)=1/2 is exact.  Also checks that dropping one order (P-1)
    would be detected."""
    d, n, P = 4, 5, 3
    rng = np.random.default_rng(3)
    qi = rng.integers(-4, 5, size=(n, d))
    ki = rng.integers(-4, 5, size=(n, d))
    vi = rng.integers(-8, 9, size=(n, 2))
    q = (qi / 8.0).astype(np.float32)                  # exact dyadic values
    k = (ki / 8.0).astype(np.float32)
    v = (vi / 4.0).astype(np.float32)

    def exact(PP):
        out = []
        for i in range(n):
            num = [Fraction(0), Fraction(0)]
            den = Fraction(0)
            for j in range(i + 1):
                x = sum(Fraction(int(qi[i, c]), 8) * Fraction(int(ki[j, c]), 8) for c in range(d)) / 2
                w = sum(x ** p / math.factorial(p) for p in range(PP))
                den += w
                for c in range(2):
                    num[c] += w * Fraction(int(vi[j, c]), 4)
            out.append([float(num[c] / den) for c in range(2)])
        return np.array(out)

    o = oracle.taylor_attention(q, k, v, P)
    e = exact(P)
    assert np.max(np.abs(o - e)) < 1e-15
    assert np.max(np.abs(oracle.taylor_attention(q, k, v, P - 1) - e)) > 1e-6


# ------------------------------------------------------------ closed forms (O6)

@pytest.mark.parametrize("d", [1, 2, 3, 5, 8, 16, 32, 64])
@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_state_size_and_flops_from_bruteforce_counts(oracle, d, P):
    """State size (d_V+1)*C(d+P-1,P-1) and the per-token FLOP formula
    (4 d_V + 2(P d + 1)/(d + 1) + 2) C(d+P-1,P-1)
    [hotdry, 'Engineering realisation of the constant compute cost'] against
    the brute-force per-order counts m_p: the FLOP formula equals
    sum_p m_p (4 d_V + 2 + 2(p+1)), the orders' update, readout, normaliser
    and two-sided expansion work."""
    if d == 64 and P == 4:
        counts = [1, 64, 2080, 45760]      # brute force at d=64, p=3 takes ~1 s
        counts[3] = len(oracle.basis_bruteforce(64, 3)[1])
    else:
        counts = [len(oracle.basis_bruteforce(d, p)[1]) for p in range(P)]
    dv = d
    assert oracle.state_size(d, dv, P) == (dv + 1) * sum(counts)
    f = oracle.flops_per_token(d, dv, P)
    assert f.denominator == 1
    assert f == sum(m * (4 * dv + 2 + 2 * (p + 1)) for p, m in enumerate(counts))


def test_flops_and_state_at_d64_p4(oracle):
    assert oracle.flops_per_token(64, 64, 4) == 12738308
    assert oracle.state_size(64, 64, 4) == 3113825
    kv, fl = oracle.conventional_cost(65536, 64, 64)
    assert kv == 8388608 and fl == 16973824


def test_page_basis_sizes_for_P3_P5_are_rejected(oracle):
    """The trade-off section prints 29635 (P=3) and 71525 (P=5) for d_K=64;
    neither is the cumulative basis size, so neither is used as a pin."""
    g = json.load(open(GOLDEN))["rejected_basis_sizes"]["page_value"]
    assert oracle.cumulative_basis(64, 3) == 2145 != g["P=3"]
    assert oracle.cumulative_basis(64, 5) == 814385 != g["P=5"]


# ------------------------------------------------------------ bf16-stored state (O8)

def test_round_bf16_matches_library_rounding(oracle):
    """O8a against torch's float32 -> bfloat16 conversion (round to nearest,
    ties to even) on random bit patterns over the whole binary32 range,
    explicit half-way cases and subnormals: bit-exact."""
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    ties = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)          # exactly half-way
    sub = rng.integers(0, 2**23, size=20000, dtype=np.uint64).astype(np.uint32)   # fp32 subnormals
    x = np.concatenate([bits, ties, sub]).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.3e38)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_integers(oracle):
    """Integers above 256 are spaced 2 apart in bf16; half-way cases go to the
    even significand."""
    got = oracle.round_bf16([255, 256, 257, 258, 259, 261, 263, 513, 515])
    assert list(got) == [255, 256, 256, 258, 260, 260, 264, 512, 516]


@pytest.mark.parametrize("d,P,n0,window", [(1, 1, 0, 1), (2, 3, 5, 1), (3, 4, 0, 1), (4, 4, 17, 1), (4, 2, 39, 1),
                                          (3, 4, 0, 4), (4, 3, 7, 16), (2, 4, 11, 5)])
def test_bf16_state_unrounded_equals_quadratic(oracle, d, P, n0, window):
    """O8 with rounding off is the one-sided recurrent form, whatever the
    split between summed prefix and steps: equal to the quadratic
    definition (O1) on rows n0.. .  Catches a wrong query weight
    (p!/alpha!, 1/p!, d^(p/2)), a step read out before its update, or a
    prefix that misses a token."""
    q, k, v = _rand_qkv(300 + 10 * d + P, (2,), 40, d, 3)
    a = oracle.bf16_state_decode(q, k, v, P, n0, rounding=False, window=window)
    b = oracle.taylor_attention(q, k, v, P)[:, n0:]
    assert a.shape == b.shape
    assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))


def test_bf16_state_exact_when_sums_are_representable(oracle):
    """With q, k in {0, +-1/2, +-1}, v in {+-1/2, +-1}, P = 3 and 12 tokens,
    every state element is a multiple of 1/8 below 12 in magnitude, which bf16
    holds exactly: the bf16-stored state must give the exact result (O1)."""
    rng = np.random.default_rng(9)
    q = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0], size=(2, 12, 4)).astype(np.float32)
    k = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0], size=(2, 12, 4)).astype(np.float32)
    v = rng.choice([0.5, -0.5, 1.0, -1.0], size=(2, 12, 3)).astype(np.float32)
    for n0 in (0, 5):
        a = oracle.bf16_state_decode(q, k, v, 3, n0)
        b = oracle.taylor_attention(q, k, v, 3)[:, n0:]
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))


@pytest.mark.parametrize("n0", [0, 300])
def test_bf16_state_count_stalls(oracle, n0):
    """P = 1 keeps the constant order: the normaliser element counts tokens.
    Stored in bf16 it stops growing where adding 1 is a half-way case that
    rounds back to the even neighbour (256 from zero; 300 stays 300 after an
    exact prefix of 300), while each step reads out from the unrounded sum
    stored + 1.  With v_0 = w and v_s = 0 after it, row s is
    w / (min(s, stall) + 1)."""
    n = 620
    w = np.array([256.0, -3.0, 0.375], dtype=np.float32)
    v = np.zeros((1, n, 3), dtype=np.float32)
    v[0, 0] = w
    q = np.zeros((1, n, 2), dtype=np.float32)
    k = np.zeros((1, n, 2), dtype=np.float32)
    o = oracle.bf16_state_decode(q, k, v, 1, n0)[0]
    stall = 256 if n0 == 0 else 300
    s = np.arange(n0, n)
    ref = w[None, :].astype(np.float64) / (np.minimum(s, stall) + 1)[:, None]
    assert np.array_equal(o, ref)
    exact = oracle.bf16_state_decode(q, k, v, 1, n0, rounding=False)[0]
    assert np.array_equal(exact, w[None, :].astype(np.float64) / (s + 1)[:, None])


@pytest.mark.parametrize("window", [4, 16])
def test_bf16_state_count_stalls_with_window(oracle, window):
    """With stores every W steps the P = 1 normaliser grows by W per store and
    stops at 256 W (adding W is then a half-way case); between stores each
    step adds its pending tokens and its own exactly, so row s reads out
    min(floor(s / W) W, 256 W) + (s mod W) + 1."""
    n = 256 * window + 3 * window + 2
    w = np.array([512.0, -1.5], dtype=np.float32)
    v = np.zeros((1, n, 2), dtype=np.float32)
    v[0, 0] = w
    q = np.zeros((1, n, 1), dtype=np.float32)
    o = oracle.bf16_state_decode(q, q, v, 1, 0, window=window)[0]
    s = np.arange(n)
    den = np.minimum((s // window) * window, 256 * window) + s % window + 1
    assert np.array_equal(o, w[None, :].astype(np.float64) / den[:, None])


# ------------------------------------------------------------ gradients (O9)

def _dyadic(rng, shape, scale=64):
    """Values k/scale with |k| <= scale: exact in fp32, and so are their sums with 2^-10."""
    return (rng.integers(-scale, scale + 1, size=shape) / scale).astype(np.float32)


@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_grad_matches_finite_differences(oracle, P):
    """O9 against central differences of O1 (the C oracle) on dyadic inputs, so
    that every perturbed value is exact in fp32: L = sum(dout * o)."""
    rng = np.random.default_rng(40 + P)
    n, d = 7, 3
    q, k, v, dout = (_dyadic(rng, (1, n, d)) for _ in range(4))
    gq, gk, gv = oracle.taylor_attention_grad(q, k, v, dout, P)
    h = 2.0 ** -10
    loss = lambda qq, kk, vv: float(np.sum(dout.astype(np.float64) * oracle.taylor_attention(qq, kk, vv, P)))
    for which, grad in ((0, gq), (1, gk), (2, gv)):
        for (i, c) in [(0, 0), (3, 1), (6, 2), (4, 0)]:
            args = [q.copy(), k.copy(), v.copy()]
            args[which][0, i, c] += h
            up = loss(*args)
            args[which][0, i, c] -= 2 * h
            dn = loss(*args)
            fd = (up - dn) / (2 * h)
            assert abs(fd - grad[0, i, c]) <= 1e-5 * max(1.0, abs(fd)), (which, i, c, fd, grad[0, i, c])


def test_grad_P1_closed_form(oracle):
    """P = 1: o_i is the running mean of v, so dv_j = sum_{i>=j} dout_i / (i + 1)
    and q, k get no gradient."""
    rng = np.random.default_rng(3)
    n, d = 20, 4
    q, k, v, dout = (rng.standard_normal((2, n, d)).astype(np.float32) for _ in range(4))
    gq, gk, gv = oracle.taylor_attention_grad(q, k, v, dout, 1)
    w = dout.astype(np.float64) / np.arange(1, n + 1)[None, :, None]
    ref = np.cumsum(w[:, ::-1], axis=1)[:, ::-1]
    assert np.max(np.abs(gv - ref)) < 1e-12
    assert np.max(np.abs(gq)) == 0 and np.max(np.abs(gk)) == 0


@pytest.mark.parametrize("P", [2, 3, 4])
def test_grad_state_form_identities(oracle, P):
    """The identities the GPU backward is built on, written out from the
    definitions: with g_i = [dout_i, -dout_i.o_i] / z_i and w' the series
    with P - 1 orders, dv_j = sum_{i>=j} w_ij g_i[:d], dk_j = sum_{i>=j}
    w'_ij ([v_j,1].g_i) q_i / sqrt d, dq_i = sum_{j<=i} w'_ij ([v_j,1].g_i)
    k_j / sqrt d.  Checked against O9."""
    rng = np.random.default_rng(50 + P)
    n, d = 30, 5
    q, k, v, dout = (rng.standard_normal((1, n, d)).astype(np.float32) for _ in range(4))
    q, k = (a / np.linalg.norm(a, axis=-1, keepdims=True) * d ** 0.25 for a in (q, k))
    q, k = q.astype(np.float32), k.astype(np.float32)
    Q, K, V, G = (a[0].astype(np.float64) for a in (q, k, v, dout))
    x = Q @ K.T / np.sqrt(d)
    w = sum(x ** p / math.factorial(p) for p in range(P))
    wd = sum(x ** p / math.factorial(p) for p in range(P - 1))
    m = np.tril(np.ones((n, n)))
    W, Wd = w * m, wd * m
    z = W.sum(1)
    o = W @ V / z[:, None]
    g = np.concatenate([G, -(G * o).sum(1, keepdims=True)], axis=1) / z[:, None]
    v1 = np.concatenate([V, np.ones((n, 1))], axis=1)
    gv_ref = W.T @ g[:, :d]
    s = g @ v1.T                      # s[i, j] = g_i . [v_j, 1]
    gk_ref = (Wd * s).T @ Q / np.sqrt(d)
    gq_ref = (Wd * s) @ K / np.sqrt(d)
    gq, gk, gv = oracle.taylor_attention_grad(q, k, v, dout, P)
    for a, b in ((gq[0], gq_ref), (gk[0], gk_ref), (gv[0], gv_ref)):
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))

# ------------------------------------------------- fp16 state with fp32 low orders (O8)

def test_round_f16_matches_library_rounding(oracle):
    """O8b against numpy's float64 -> float16 conversion (IEEE round to nearest,
    ties to even) on random values over binary16's whole range, exact half-way
    cases of normal and subnormal spacing, and the overflow edge: bit-exact."""
    rng = np.random.default_rng(15)
    e = rng.integers(-30, 17, size=200000)
    x = rng.uniform(1.0, 2.0, size=e.size) * np.exp2(e) * rng.choice([-1.0, 1.0], size=e.size)
    m = rng.integers(0, 1024, size=20000)
    ee = rng.integers(-14, 16, size=m.size)
    ties = (1024 + m + 0.5) * np.exp2(ee - 10.0)                 # half-way between normal neighbours
    sub_ties = (rng.integers(0, 1024, size=5000) + 0.5) * 2.0 ** -24   # half-way in the subnormal range
    edge = np.array([65504.0, 65519.99, 65520.0, 65536.0, -65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26])
    x = np.concatenate([x, ties, -ties, sub_ties, edge])
    with np.errstate(over="ignore"):                            # the overflow edge becomes inf
        ref = x.astype(np.float16).astype(np.float64)
    got = oracle.round_f16(x)
    assert np.array_equal(got, ref)


def test_round_f16_integers(oracle):
    """Integers above 2048 are spaced 2 apart in binary16; half-way cases go to
    the even significand."""
    got = oracle.round_f16([2047, 2048, 2049, 2050, 2051, 2053, 4097, 4099, 4101])
    assert list(got) == [2047, 2048, 2048, 2050, 2052, 2052, 4096, 4100, 4100]


@pytest.mark.parametrize("low_orders", [0, 1])
def test_f16_state_count_stalls_only_in_fp16(oracle, low_orders):
    """P = 1: the normaliser element counts tokens.  In fp16 (low_orders 0) it
    stops at 2048, where adding 1 is a half-way case that rounds back to the
    even neighbour; with order 0 in fp32 (low_orders 1) it counts on exactly.
    With v_0 = w and v_s = 0 after it, row s is w / (count + 1)."""
    n = 2200
    w = np.array([2048.0, -3.0, 0.375], dtype=np.float32)
    v = np.zeros((1, n, 3), dtype=np.float32)
    v[0, 0] = w
    q = np.zeros((1, n, 2), dtype=np.float32)
    o = oracle.f16_state_decode(q, q, v, 1, 0, low_orders=low_orders)[0]
    s = np.arange(n)
    count = np.minimum(s, 2048) if low_orders == 0 else s
    assert np.array_equal(o, w[None, :].astype(np.float64) / (count + 1)[:, None])


@pytest.mark.parametrize("d,P,n0", [(2, 3, 5), (4, 4, 17), (3, 2, 0)])
def test_f16_state_all_fp32_is_fp32_close(oracle, d, P, n0):
    """With every order stored in fp32 (low_orders = P) the only error is one
    binary32 rounding per element per store: within 1e-5 of O1."""
    q, k, v = _rand_qkv(700 + 10 * d + P, (2,), 60, d, 3)
    a = oracle.f16_state_decode(q, k, v, P, n0, low_orders=P)
    b = oracle.taylor_attention(q, k, v, P)[:, n0:]
    assert np.max(np.abs(a - b)) <= 1e-5 * np.max(np.abs(b))


def _state16_numpy(q, k, v, P, n0, low_features, window):
    """Brute-force reading of the fp16 state with numpy's own roundings: tuples
    by itertools, exact (fp64) prefix sums stored rounded, each step adds its
    pending tokens exactly, reads out, and every window-th step stores rounded
    (fp32 for the first low_features features, numbered order by order, fp16
    for the rest)."""
    import itertools
    n, d = q.shape[0], q.shape[1]
    dv = v.shape[1]
    feats = [(p, t) for p in range(P) for t in itertools.combinations_with_replacement(range(d), p)]

    def mono(x, t):
        return float(np.prod([float(x[i]) for i in t])) if t else 1.0

    def weight(p, t):   # p!/alpha! / (p! d^(p/2)) = 1 / (alpha! d^(p/2))
        alpha = np.prod([math.factorial(t.count(i)) for i in set(t)]) if t else 1
        return 1.0 / (alpha * d ** (p / 2))

    def rnd(i, x):
        return float(np.float32(x)) if i < low_features else float(np.float16(x))

    vv = lambda s, c: float(v[s, c]) if c < dv else 1.0
    S = [[rnd(i, sum(mono(k[s], t) * vv(s, c) for s in range(n0))) for c in range(dv + 1)]
         for i, (p, t) in enumerate(feats)]
    out, first = [], n0
    for s in range(n0, n):
        store = s - first + 1 >= window
        y = np.zeros(dv + 1)
        for i, (p, t) in enumerate(feats):
            mq = weight(p, t) * mono(q[s], t)
            for c in range(dv + 1):
                x = S[i][c] + sum(mono(k[u], t) * vv(u, c) for u in range(first, s + 1))
                y[c] += mq * x
                if store:
                    S[i][c] = rnd(i, x)
        if store:
            first = s + 1
        out.append(y[:dv] / y[dv])
    return np.array(out)


@pytest.mark.parametrize("low_orders,low_features,window", [(0, 0, 1), (1, 1, 1), (2, 3, 1), (2, 3, 3), (None, 5, 1)])
def test_f16_state_matches_numpy_emulation(oracle, low_orders, low_features, window):
    """O8 (fp16 with fp32 low orders) against the brute-force numpy reading on
    a case whose sums fp16 cannot hold exactly (large v), d = 2, P = 3 (1 + 2 + 3
    features): the orders below low_orders, or the first low_features features
    (5 cuts inside order 2), in fp32.  Equal to fp64 rounding; and another cut
    gives a different result."""
    rng = np.random.default_rng(21 + low_features)
    n, d, P, n0 = 14, 2, 3, 4
    q = rng.normal(size=(1, n, d)).astype(np.float32)
    k = rng.normal(size=(1, n, d)).astype(np.float32)
    v = (rng.normal(size=(1, n, 2)) * 300).astype(np.float32)
    if low_orders is None:
        a = oracle.f16_state_decode(q, k, v, P, n0, window=window, low_features=low_features)[0]
    else:
        a = oracle.f16_state_decode(q, k, v, P, n0, low_orders=low_orders, window=window)[0]
    b = _state16_numpy(q[0], k[0], v[0], P, n0, low_features, window)
    assert np.max(np.abs(a - b)) <= 1e-9 * np.max(np.abs(b))
    other = oracle.f16_state_decode(q, k, v, P, n0, window=window, low_features=6 if low_features < 3 else 0)[0]
    assert np.max(np.abs(other - a)) > 1e-6 * np.max(np.abs(b))
