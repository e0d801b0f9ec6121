"""Pins specific to the C++ oracle (``oracle.cpp``).

* It agrees with the numpy implementation of the same definitions on random
  shapes that exercise every argument: GQA, Nq != Nk, dv != d, row subsets,
  several row panels (N > 1024), ragged and empty sequences.
* Its result does not depend on the OpenMP thread count (bitwise).
* Its multiply-add counter -- incremented by the product loops as they run --
  equals a brute-force count of the visible (query, key) pairs, and the FLOP
  convention functions are pinned against that count: two products of one
  multiply-add per visible pair and d for the forward (ledger page, "FLOPs"
  section: 4 n^2 d per head), five for the backward, two for HSTU; causal is
  counted as half of the full count (HSTU page, optimisation two).
"""

import numpy as np
import pytest

import oracle
from oracle import cpp, numpy_ref


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def visible_pairs(nq, nk, causal):
    """Brute force: number of (i, j) with key j visible from row i."""
    return sum(min(i + 1, nk) if causal else nk for i in range(nq))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,dv", [(2, 4, 2, 37, 37, 16, 16), (1, 3, 1, 20, 45, 8, 5),
                                                (1, 2, 2, 45, 20, 8, 12), (1, 1, 1, 1500, 1500, 4, 3)])
def test_forward_matches_numpy(causal, B, H, Hkv, Nq, Nk, d, dv):
    q, k, v = rnd(1, B, H, Nq, d), rnd(2, B, Hkv, Nk, d), rnd(3, B, Hkv, Nk, dv)
    O1, L1 = cpp.attention_forward(q, k, v, 0.4, causal)
    O2, L2 = numpy_ref.attention_forward(q, k, v, 0.4, causal)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-12)
    rows = np.array([0, Nq // 3, Nq - 1])
    O3, L3 = cpp.attention_forward(q, k, v, 0.4, causal, rows=rows)
    assert np.array_equal(O3, O1[:, :, rows]) and np.array_equal(L3, L1[:, :, rows])


def test_panels_span_long_rows():
    """N > 1024 splits rows into panels of 2^20 / N rows; the panel
    boundaries must not show in the result (rows are independent)."""
    N, d = 2100, 4  # panels of 499 rows: boundaries at 499, 998, 1497, 1996
    q, k, v = rnd(4, 1, 1, N, d), rnd(5, 1, 1, N, d), rnd(6, 1, 1, N, d)
    O, L = cpp.attention_forward(q, k, v, 0.5, True)
    for i in (498, 499, 500, 1996, 2099):
        Oi, Li = cpp.attention_forward(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.5, False)
        np.testing.assert_allclose(O[0, 0, i], Oi[0, 0, 0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[0, 0, i], Li[0, 0, 0], rtol=0, atol=1e-13)


def test_decode_and_paged_match_numpy():
    from synthgen import bf16_bits_to_f64 as f
    from synthgen import workloads as W

    c = W.Decode("cpp_pin", 4, 8, 2, 300, 128, 0.0884, 1, 300, 12)
    x = W.decode_inputs(c, seqlens=[0, 1, 299, 300])
    O1, L1 = cpp.decode(f(x.q), f(x.k), f(x.v), x.seqlens, c.scale)
    O2, L2 = numpy_ref.decode(f(x.q), f(x.k), f(x.v), x.seqlens, c.scale)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-14)
    assert np.array_equal(np.isneginf(L1), np.isneginf(L2))
    fin = np.isfinite(L2)
    np.testing.assert_allclose(L1[fin], L2[fin], rtol=0, atol=1e-13)
    px = W.paged_from_decode(x, 32)
    O3, L3 = cpp.decode_paged(f(x.q), f(px.k_pages), f(px.v_pages), px.block_table, x.seqlens, c.scale)
    assert np.array_equal(O3, O1) and np.array_equal(L3, L1)


@pytest.mark.parametrize("causal", [False, True])
def test_hstu_jagged_matches_numpy(causal):
    lengths = [5, 0, 1, 1100, 7]
    off = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = int(off[-1]), 2, 8
    q, k, v = rnd(7, T, H, d), rnd(8, T, H, d), rnd(9, T, H, 6)
    O1 = cpp.hstu_jagged(q, k, v, off, 0.3, 1 / 50, causal)
    O2 = numpy_ref.hstu_jagged(q, k, v, off, 0.3, 1 / 50, causal)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_numpy(causal):
    B, H, Hkv, N, d = 2, 4, 2, 41, 8
    q, k, v, do = rnd(10, B, H, N, d), rnd(11, B, Hkv, N, d), rnd(12, B, Hkv, N, d), rnd(13, B, H, N, d)
    for a, b in zip(cpp.attention_backward(q, k, v, do, 0.35, causal),
                    numpy_ref.attention_backward(q, k, v, do, 0.35, causal)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_result_does_not_depend_on_thread_count():
    q, k, v = rnd(14, 2, 4, 300, 16), rnd(15, 2, 2, 300, 16), rnd(16, 2, 2, 300, 16)
    jq, jk, jv = rnd(27, 300, 4, 16), rnd(28, 300, 4, 16), rnd(29, 300, 4, 16)

    def run():
        out = list(cpp.attention_forward(q, k, v, 0.3, True))
        out += list(cpp.attention_backward(q, k, v, q, 0.3, True))
        out.append(cpp.hstu_jagged(jq, jk, jv, [0, 100, 300], 0.5, 0.1, True))
        return out

    n0 = cpp.max_threads()
    try:
        cpp.set_threads(1)
        one = run()
        cpp.set_threads(max(n0, 4))
        many = run()
    finally:
        cpp.set_threads(n0)
    for a, b in zip(one, many):
        assert np.array_equal(a, b)


# --- FLOP convention against the executed multiply-adds -------------------------

@pytest.mark.parametrize("n,d", [(1, 1), (5, 3), (16, 8), (33, 64), (1200, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_flops_against_counted_macs(n, d, causal):
    B, H = 2, 3
    counts = {}
    cpp.attention_forward(rnd(17, B, H, n, d), rnd(18, B, H, n, d), rnd(19, B, H, n, d), 0.2, causal,
                          counts=counts)
    pairs = visible_pairs(n, n, causal)
    assert counts["macs"] == B * H * 2 * d * pairs  # QK^T and PV: d multiply-adds per visible pair each
    full = oracle.attention_flops(B, H, n, d, False)
    if not causal:
        assert full == 2 * counts["macs"]
    else:
        # the convention halves the full count; the executed count exceeds that
        # by the diagonal's n/2 pairs per head, 2 n d FLOP over the two products
        assert oracle.attention_flops(B, H, n, d, True) == full // 2
        assert oracle.attention_flops(B, H, n, d, True) == 2 * counts["macs"] - B * H * 2 * n * d


def test_decode_macs_count_every_valid_row_once():
    from synthgen import bf16_bits_to_f64 as f
    from synthgen import workloads as W

    c = W.Decode("cpp_macs", 3, 8, 2, 100, 128, 0.0884, 1, 100, 13)
    x = W.decode_inputs(c, seqlens=[0, 17, 100])
    counts = {}
    cpp.decode(f(x.q), f(x.k), f(x.v), x.seqlens, c.scale, counts=counts)
    assert counts["macs"] == c.H * 2 * c.d * int(np.sum(x.seqlens))


@pytest.mark.parametrize("n,d", [(1, 4), (7, 3), (40, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_flops_against_counted_macs(n, d, causal):
    B, H, Hkv = 1, 4, 2
    counts = {}
    cpp.attention_backward(rnd(20, B, H, n, d), rnd(21, B, Hkv, n, d), rnd(22, B, Hkv, n, d),
                           rnd(23, B, H, n, d), 0.3, causal, counts=counts)
    pairs = visible_pairs(n, n, causal)
    # five products (S, dP, dQ, dV, dK), d multiply-adds per visible pair each
    assert counts["macs"] == B * H * 5 * d * pairs
    if not causal:
        assert oracle.attention_bwd_flops(B, H, n, d, False) == 2 * counts["macs"]
    else:
        assert oracle.attention_bwd_flops(B, H, n, d, True) == 2 * counts["macs"] - B * H * 5 * n * d


@pytest.mark.parametrize("causal", [False, True])
def test_hstu_flops_against_counted_macs(causal):
    lengths = [3, 0, 1, 64, 17]
    off = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = int(off[-1]), 3, 8
    counts = {}
    cpp.hstu_jagged(rnd(24, T, H, d), rnd(25, T, H, d), rnd(26, T, H, d), off, 0.5, 0.1, causal, counts=counts)
    pairs = sum(visible_pairs(L, L, causal) for L in lengths)
    assert counts["macs"] == H * 2 * d * pairs
    if not causal:
        assert oracle.hstu_flops(lengths, H, d, False) == 2 * counts["macs"]
    else:
        assert oracle.hstu_flops(lengths, H, d, True) == 2 * counts["macs"] - H * 2 * d * sum(lengths)
