"""Pins of the paged-cache decode oracle (``oracle.decode_paged``).

The page scatter used here (``synthgen.workloads.paged_from_decode``) is
independent of the oracle's gather: a wrong page order, axis or row count in
either shows up as a difference from decode on the contiguous cache.
"""

import numpy as np
import pytest

import oracle
from synthgen import bf16_bits_to_f64
from synthgen import workloads as W


# run against both implementations: the C++ oracle and the numpy one
IMPLS = {"cpp": oracle.cpp, "numpy": oracle.numpy_ref}


@pytest.fixture(params=sorted(IMPLS))
def orc(request):
    return IMPLS[request.param]


def _case(seqlens, Lmax=200, H=8, Hkv=2):
    c = W.Decode("paged_pin", len(seqlens), H, Hkv, Lmax, 128, 0.0884, 1, Lmax, 11)
    return W.decode_inputs(c, seqlens=seqlens)


@pytest.mark.parametrize("P", [16, 32, 64, 256])
def test_paged_decode_equals_contiguous_decode(orc, P):
    x = _case([1, 37, 200, 128])
    px = W.paged_from_decode(x, P, perm_seed=P)
    f = bf16_bits_to_f64
    O1, L1 = orc.decode(f(x.q), f(x.k), f(x.v), x.seqlens, x.case.scale)
    O2, L2 = orc.decode_paged(f(x.q), f(px.k_pages), f(px.v_pages), px.block_table, x.seqlens, x.case.scale)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    # the physical order really is shuffled
    assert not np.array_equal(px.block_table.reshape(-1), np.arange(px.block_table.size))


def test_paged_decode_identity_table_reads_pages_in_order(orc):
    x = _case([50, 200])
    px = W.paged_from_decode(x, 16, spare_pages=0)
    # re-lay the pages in logical order and use the identity table
    kp = px.k_pages[px.block_table.reshape(-1)]
    vp = px.v_pages[px.block_table.reshape(-1)]
    table = np.arange(px.block_table.size, dtype=np.int32).reshape(px.block_table.shape)
    f = bf16_bits_to_f64
    O1, L1 = orc.decode(f(x.q), f(x.k), f(x.v), x.seqlens, x.case.scale)
    O2, L2 = orc.decode_paged(f(x.q), f(kp), f(vp), table, x.seqlens, x.case.scale)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_empty_history_gives_zero_output_and_minus_inf_lse(orc):
    x = _case([0, 5])
    px = W.paged_from_decode(x, 16)
    f = bf16_bits_to_f64
    for O, L in (orc.decode(f(x.q), f(x.k), f(x.v), x.seqlens, 0.1),
                 orc.decode_paged(f(x.q), f(px.k_pages), f(px.v_pages), px.block_table, x.seqlens, 0.1)):
        assert np.all(O[0] == 0.0) and np.all(np.isneginf(L[0]))
        assert np.all(np.isfinite(O[1])) and np.all(np.isfinite(L[1]))
