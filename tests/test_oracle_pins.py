"""Pins for the fp64 oracle: closed forms, invariants and library routines.

Each test ties the oracle to something other than itself, chosen so that a
plausible slip (a dropped term, a wrong sign or index, a transposed operand,
a wrong log base, a wrong mask) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from synthgen import bf16_bits_to_f64, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# The pins run against both implementations of the definitions: the C++ oracle
# (the reference the GPU is checked against) and the numpy one.
IMPLS = {"cpp": oracle.cpp, "numpy": oracle.numpy_ref}


@pytest.fixture(params=sorted(IMPLS))
def orc(request):
    return IMPLS[request.param]


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# --- softmax attention -----------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(orc, causal):
    q, k = rnd(1, 96, 16), rnd(2, 96, 16)
    P = orc.attention_probs(q, k, 0.25, causal)
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    if causal:
        assert np.all(np.triu(P, 1) == 0)
        assert np.all(np.diag(P) > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_match_scipy_softmax(orc, causal):
    q, k = rnd(3, 40, 8), rnd(4, 40, 8)
    scale = 0.7
    S = scale * (q @ k.T)
    if causal:
        S = np.where(np.tril(np.ones_like(S)) > 0, S, -np.inf)
    np.testing.assert_allclose(orc.attention_probs(q, k, scale, causal),
                               scipy.special.softmax(S, axis=1), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (4, 2), (6, 1)])
def test_forward_matches_torch_sdpa_fp64(orc, causal, H, Hkv):
    """Library routine: torch's scaled_dot_product_attention on the CPU in fp64."""
    B, N, d, scale = 2, 37, 16, 0.3
    q, k, v = rnd(5, B, H, N, d), rnd(6, B, Hkv, N, d), rnd(7, B, Hkv, N, d)
    O, L = orc.attention_forward(q, k, v, scale, causal)
    rep = H // Hkv
    kt = torch.from_numpy(k).repeat_interleave(rep, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(rep, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, vt, is_causal=causal, scale=scale).numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-13)
    # LSE against scipy's logsumexp of the scaled, masked scores.
    S = scale * np.einsum("bhnd,bhmd->bhnm", q, kt.numpy())
    if causal:
        S = np.where(np.tril(np.ones((N, N))) > 0, S, -np.inf)
    np.testing.assert_allclose(L, scipy.special.logsumexp(S, axis=-1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(orc, causal):
    N, d, scale = 50, 12, 0.4
    q = rnd(8, 1, 1, N, d)
    krow = rnd(9, d)
    k = np.broadcast_to(krow, (1, 1, N, d)).copy()
    v = rnd(10, 1, 1, N, d)
    O, L = orc.attention_forward(q, k, v, scale, causal)
    for i in range(N):
        n_vis = i + 1 if causal else N
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, :n_vis].mean(axis=0), rtol=0, atol=1e-13)
        s = scale * q[0, 0, i] @ krow
        assert abs(L[0, 0, i] - (s + math.log(n_vis))) < 1e-13 * max(1.0, abs(s) + 5)


def test_causal_row_zero_is_v0(orc):
    q, k, v = rnd(11, 1, 3, 20, 8), rnd(12, 1, 3, 20, 8), rnd(13, 1, 3, 20, 8)
    O, L = orc.attention_forward(q, k, v, 0.5, True)
    assert np.array_equal(O[0, :, 0], v[0, :, 0])
    np.testing.assert_allclose(L[0, :, 0], 0.5 * np.einsum("hd,hd->h", q[0, :, 0], k[0, :, 0]),
                               rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 3, 64, 100])
def test_online_equals_two_pass(orc, causal, block):
    N, d, scale = 100, 16, 0.35
    q, k, v = rnd(14, N, d) * 2, rnd(15, N, d) * 2, rnd(16, N, d)
    O2, L2 = orc.attention_forward(q[None, None], k[None, None], v[None, None], scale, causal)
    O1, L1 = oracle.attention_online(q, k, v, scale, causal, block)
    np.testing.assert_allclose(O1, O2[0, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L1, L2[0, 0], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_extract_probabilities(orc, causal):
    N = 24
    q, k = rnd(17, N, 6), rnd(18, N, 6)
    v = np.eye(N)
    O, _ = orc.attention_forward(q[None, None], k[None, None], v[None, None], 0.9, causal)
    np.testing.assert_allclose(O[0, 0], orc.attention_probs(q, k, 0.9, causal), rtol=0, atol=1e-14)


def test_two_keys_is_a_sigmoid(orc):
    q, k, v = rnd(19, 7, 5), rnd(20, 2, 5), rnd(21, 2, 3)
    scale = 0.8
    O, _ = orc.attention_forward(q[None, None], k[None, None], v[None, None], scale, False)
    s = scale * (q @ k.T)
    p0 = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))
    expect = p0[:, None] * v[0] + (1 - p0)[:, None] * v[1]
    np.testing.assert_allclose(O[0, 0], expect, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_uniform_weights(orc, causal):
    N = 33
    q, k, v = rnd(22, 1, 1, N, 4), rnd(23, 1, 1, N, 4), rnd(24, 1, 1, N, 4)
    O, L = orc.attention_forward(q, k, v, 0.0, causal)
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    expect = np.cumsum(v[0, 0], axis=0) / counts[:, None] if causal else np.broadcast_to(v[0, 0].mean(0), (N, 4))
    np.testing.assert_allclose(O[0, 0], expect, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[0, 0], np.log(counts), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_row_shift_invariance_without_overflow(orc, causal):
    """Adding the same large constant to every score of a row changes only LSE."""
    N, d, scale = 30, 8, 0.5
    q, k, v = rnd(25, N, d), rnd(26, N, d), rnd(27, N, d)
    c = 2.0e4  # scale * c = 1e4: exp(1e4) would overflow without the max shift
    q2 = np.concatenate([q, np.full((N, 1), c)], axis=1)
    k2 = np.concatenate([k, np.ones((N, 1))], axis=1)
    O1, L1 = orc.attention_forward(q[None, None], k[None, None], v[None, None], scale, causal)
    O2, L2 = orc.attention_forward(q2[None, None], k2[None, None], v[None, None], scale, causal)
    assert np.all(np.isfinite(O2)) and np.all(np.isfinite(L2))
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-11)
    np.testing.assert_allclose(L2 - L1, scale * c, rtol=1e-12)


def test_key_permutation_invariance(orc):
    N, d = 40, 8
    q, k, v = rnd(28, N, d), rnd(29, N, d), rnd(30, N, d)
    perm = np.random.default_rng(31).permutation(N)
    O1, L1 = orc.attention_forward(q[None, None], k[None, None], v[None, None], 0.3, False)
    O2, L2 = orc.attention_forward(q[None, None], k[perm][None, None], v[perm][None, None], 0.3, False)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=1e-13)


def test_causality_future_rows_do_not_matter(orc):
    N, d, i0 = 40, 8, 17
    q, k, v = rnd(32, N, d), rnd(33, N, d), rnd(34, N, d)
    k2, v2 = k.copy(), v.copy()
    k2[i0 + 1:] = rnd(35, N - i0 - 1, d) * 10
    v2[i0 + 1:] = rnd(36, N - i0 - 1, d) * 10
    O1, L1 = orc.attention_forward(q[None, None], k[None, None], v[None, None], 0.3, True)
    O2, L2 = orc.attention_forward(q[None, None], k2[None, None], v2[None, None], 0.3, True)
    assert np.array_equal(O1[0, 0, :i0 + 1], O2[0, 0, :i0 + 1])
    assert np.array_equal(L1[0, 0, :i0 + 1], L2[0, 0, :i0 + 1])
    assert not np.allclose(O1[0, 0, i0 + 1:], O2[0, 0, i0 + 1:])


def test_gqa_equals_repeated_heads(orc):
    B, H, Hkv, N, d = 2, 8, 2, 19, 8
    q, k, v = rnd(37, B, H, N, d), rnd(38, B, Hkv, N, d), rnd(39, B, Hkv, N, d)
    O1, L1 = orc.attention_forward(q, k, v, 0.4, True)
    O2, L2 = orc.attention_forward(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.4, True)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-15)


def test_row_subset_equals_full(orc):
    B, H, N, d = 1, 2, 70, 8
    q, k, v = rnd(40, B, H, N, d), rnd(41, B, H, N, d), rnd(42, B, H, N, d)
    rows = np.array([0, 5, 31, 69])
    O, L = orc.attention_forward(q, k, v, 0.3, True)
    Os, Ls = orc.attention_forward(q, k, v, 0.3, True, rows=rows)
    np.testing.assert_allclose(Os, O[:, :, rows], rtol=0, atol=1e-15)
    np.testing.assert_allclose(Ls, L[:, :, rows], rtol=0, atol=1e-15)


def test_lse_combine_of_key_chunks_recovers_full_result(orc):
    """logsumexp over per-chunk LSEs equals the full LSE, and the chunk
    outputs weighted by exp(lse_c - lse) sum to the full output."""
    N, d, scale = 90, 8, 0.45
    q, k, v = rnd(43, 5, d), rnd(44, N, d), rnd(45, N, d)
    O, L = orc.attention_forward(q[None, None], k[None, None], v[None, None], scale, False)
    bounds = [0, 7, 40, 41, 90]
    parts = [orc.attention_forward(q[None, None], k[None, None, a:b], v[None, None, a:b], scale, False)
             for a, b in zip(bounds[:-1], bounds[1:])]
    lse_c = np.stack([p[1][0, 0] for p in parts])
    o_c = np.stack([p[0][0, 0] for p in parts])
    lse = scipy.special.logsumexp(lse_c, axis=0)
    np.testing.assert_allclose(lse, L[0, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose((np.exp(lse_c - lse)[..., None] * o_c).sum(0), O[0, 0], rtol=0, atol=1e-13)


# --- decode ------------------------------------------------------------------

def test_decode_equals_last_row_of_causal_prefill(orc):
    B, H, Hkv, Lmax, d = 3, 4, 2, 30, 8
    k, v = rnd(46, B, Hkv, Lmax, d), rnd(47, B, Hkv, Lmax, d)
    seqlens = np.array([30, 1, 17])
    q = rnd(48, B, H, d)
    O, L = orc.decode(q, k, v, seqlens, 0.35)
    for b in range(B):
        n = seqlens[b]
        qq = np.zeros((1, H, n, d))
        qq[0, :, n - 1] = q[b]
        Of, Lf = orc.attention_forward(qq, k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.35, True, rows=[n - 1])
        np.testing.assert_allclose(O[b], Of[0, :, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[b], Lf[0, :, 0], rtol=0, atol=1e-13)


def test_decode_never_reads_beyond_length(orc):
    B, H, Hkv, Lmax, d = 2, 2, 1, 16, 4
    k, v = rnd(49, B, Hkv, Lmax, d), rnd(50, B, Hkv, Lmax, d)
    seqlens = np.array([5, 16])
    k[0, :, 5:] = np.nan
    v[0, :, 5:] = np.nan
    O, L = orc.decode(rnd(51, B, H, d), k, v, seqlens, 0.5)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))


def test_decode_single_key_returns_its_value(orc):
    k, v = rnd(52, 1, 1, 8, 4), rnd(53, 1, 1, 8, 4)
    q = rnd(54, 1, 3, 4)
    O, L = orc.decode(q, k, v, np.array([1]), 0.5)
    for h in range(3):
        assert np.array_equal(O[0, h], v[0, 0, 0])
        assert abs(L[0, h] - 0.5 * q[0, h] @ k[0, 0, 0]) < 1e-15


# --- HSTU ----------------------------------------------------------------------

def test_silu_matches_library():
    x = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(oracle.silu(x), x * scipy.special.expit(x), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(oracle.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(),
                               rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def test_hstu_zero_query_gives_zero(orc):
    q = np.zeros((9, 4))
    O = orc.hstu_dense(q, rnd(55, 9, 4), rnd(56, 9, 4), 0.3, 0.1, True)
    assert np.all(O == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_hstu_identical_keys_closed_form(orc, causal):
    """With every key equal, row i's score is alpha * q_i.k for all visible j,
    so O_i = inv_n * silu(alpha q_i.k) * (sum of the visible v_j)."""
    L, d, alpha, inv_n = 21, 6, 0.37, 1.0 / 7.0
    q, v = rnd(57, L, d) * 3, rnd(58, L, d)
    krow = rnd(59, d)
    k = np.broadcast_to(krow, (L, d))
    O = orc.hstu_dense(q, k, v, alpha, inv_n, causal)
    x = alpha * (q @ krow)
    y = x * scipy.special.expit(x)
    vs = np.cumsum(v, axis=0) if causal else np.broadcast_to(v.sum(0), (L, d))
    np.testing.assert_allclose(O, inv_n * y[:, None] * vs, rtol=0, atol=1e-13)


def test_hstu_single_pair_closed_form(orc):
    """Two tokens, causal: row 0 sees itself only; row 1 sees both."""
    q, k, v = rnd(60, 2, 3), rnd(61, 2, 3), rnd(62, 2, 3)
    a, n = 0.9, 0.25
    O = orc.hstu_dense(q, k, v, a, n, True)
    def f(x):
        return x / (1 + math.exp(-x))
    np.testing.assert_allclose(O[0], n * f(a * q[0] @ k[0]) * v[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O[1], n * (f(a * q[1] @ k[0]) * v[0] + f(a * q[1] @ k[1]) * v[1]),
                               rtol=0, atol=1e-15)


def test_hstu_jagged_equals_each_sequence_alone(orc):
    lengths = [5, 0, 1, 13, 7]
    off = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = off[-1], 3, 4
    q, k, v = rnd(63, T, H, d), rnd(64, T, H, d), rnd(65, T, H, d)
    O = orc.hstu_jagged(q, k, v, off, 0.5, 0.2, True)
    for b in range(len(lengths)):
        s, e = off[b], off[b + 1]
        for h in range(H):
            assert np.array_equal(O[s:e, h], orc.hstu_dense(q[s:e, h], k[s:e, h], v[s:e, h], 0.5, 0.2, True))
    # no cross-sequence terms: changing sequence 3 leaves the others unchanged
    k2 = k.copy()
    k2[off[3]:off[4]] += 1.0
    O2 = orc.hstu_jagged(q, k2, v, off, 0.5, 0.2, True)
    keep = np.ones(T, bool)
    keep[off[3]:off[4]] = False
    assert np.array_equal(O[keep], O2[keep])


# --- FLOP convention and the pages' printed figures ------------------------------

def _brute_force_macs(n, d, causal):
    """Count multiply-adds of QK^T and PV restricted to the visible pairs."""
    pairs = sum(len(oracle.allowed_keys(i, n, causal)) for i in range(n))
    return 2 * pairs * d


@pytest.mark.parametrize("n,d", [(1, 1), (5, 3), (16, 8), (33, 64)])
def test_flop_convention(n, d):
    assert oracle.attention_flops(1, 1, n, d, False) == 2 * _brute_force_macs(n, d, False)
    # Causal convention is half of the full count; the exact visible-pair count
    # n(n+1)/2 exceeds n^2/2 by the diagonal, n/2 pairs, i.e. 2nd FLOPs over
    # the two products.
    assert oracle.attention_flops(1, 1, n, d, True) == 2 * _brute_force_macs(n, d, True) - 2 * n * d
    assert oracle.attention_flops(3, 5, n, d, True) == 15 * oracle.attention_flops(1, 1, n, d, True)


def test_page_figures(orc):
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        figs = json.load(f)
    led = figs["ledger_flops"]
    d = led["d_model"]
    n0 = led["crossover_n"]
    # Attention FLOPs 4n^2 d against the FFN's 16 n d^2: equal at n = 4d.
    assert oracle.attention_flops(1, 1, n0, d, False) == 16 * n0 * d * d
    assert oracle.attention_flops(1, 1, n0 + 1, d, False) > 16 * (n0 + 1) * d * d
    assert oracle.attention_flops(1, 1, n0 - 1, d, False) < 16 * (n0 - 1) * d * d
    sc = figs["score_matrix_4096"]
    P = orc.attention_probs(np.zeros((sc["n"], 1)), np.zeros((sc["n"], 1)), 1.0, False)
    assert P.size == sc["elements"]
    assert P.size * 4 == sc["fp32_bytes"]


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e38, np.inf, -0.0], dtype=np.float32)
    got = bf16_bits_to_f64(f32_to_bf16_bits(x))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    r = np.random.default_rng(66).standard_normal(100000).astype(np.float32) * 10
    assert np.array_equal(bf16_bits_to_f64(f32_to_bf16_bits(r)),
                          torch.from_numpy(r).to(torch.bfloat16).to(torch.float64).numpy())


# --- brute force in extended precision ---------------------------------------

def _brute_attention(q, k, v, scale, causal):
    """Nested loops in extended precision, written from the definition:
    s_ij = scale q_i.k_j over visible j, m_i = max, l_i = sum exp(s - m),
    O_i = sum exp(s - m) v_j / l_i, LSE_i = m_i + ln l_i."""
    ld = np.longdouble
    n, d = q.shape
    O = np.zeros((n, v.shape[1]), dtype=ld)
    L = np.zeros(n, dtype=ld)
    for i in range(n):
        js = list(range(i + 1)) if causal else list(range(k.shape[0]))
        s = []
        for j in js:
            acc = ld(0)
            for c in range(d):
                acc += ld(q[i, c]) * ld(k[j, c])
            s.append(ld(scale) * acc)
        m = max(s)
        w = [np.exp(x - m) for x in s]
        tot = sum(w)
        for t, j in enumerate(js):
            for c in range(v.shape[1]):
                O[i, c] += w[t] / tot * ld(v[j, c])
        L[i] = m + np.log(tot)
    return O, L


@pytest.mark.parametrize("n", [1, 5, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_extended_precision_brute_force(orc, n, causal):
    q, k, v = rnd(90 + n, n, 8), rnd(91 + n, n, 8), rnd(92 + n, n, 6)
    scale = 0.37
    O, L = orc.attention_forward(q[None, None], k[None, None], v[None, None], scale, causal)
    Ob, Lb = _brute_attention(q, k, v, scale, causal)
    np.testing.assert_allclose(O[0, 0], Ob.astype(np.float64), rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[0, 0], Lb.astype(np.float64), rtol=0, atol=1e-13)


def _brute_hstu(q, k, v, alpha, inv_n, causal):
    """HSTU in extended precision with loops: x = alpha q_i.k_j,
    y = x / (1 + e^-x) over visible j, O_i = inv_n sum y v_j."""
    ld = np.longdouble
    n, d = q.shape
    O = np.zeros((n, v.shape[1]), dtype=ld)
    for i in range(n):
        for j in (range(i + 1) if causal else range(n)):
            x = ld(0)
            for c in range(d):
                x += ld(q[i, c]) * ld(k[j, c])
            x *= ld(alpha)
            y = x / (ld(1) + np.exp(-x))
            for c in range(v.shape[1]):
                O[i, c] += ld(inv_n) * y * ld(v[j, c])
    return O


@pytest.mark.parametrize("n", [1, 6, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_hstu_matches_extended_precision_brute_force(orc, n, causal):
    q, k, v = rnd(93 + n, n, 8), rnd(94 + n, n, 8), rnd(95 + n, n, 5)
    O = orc.hstu_dense(q, k, v, 0.6, 0.125, causal)
    np.testing.assert_allclose(O, _brute_hstu(q, k, v, 0.6, 0.125, causal).astype(np.float64), rtol=0, atol=1e-14)
