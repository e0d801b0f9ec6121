"""The benchmark's FLOP and byte conventions (CPU).

``bench.py`` computes its throughput figures with its own small formulas (it
may not import the oracle outside its CPU-baseline leg).  These tests pin
them to the oracle's convention functions, which are themselves pinned to the
multiply-adds the C++ oracle's loops execute (``tests/test_oracle_cpp.py``).
"""

import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("B,H,N,d", [(8, 32, 4096, 128), (1, 32, 4096, 64), (1, 32, 32768, 128), (2, 3, 17, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_and_backward_flops(B, H, N, d, causal):
    assert bench.prefill_flops(B, H, N, d, causal) == oracle.attention_flops(B, H, N, d, causal)
    assert bench.backward_flops(B, H, N, d, causal) == oracle.attention_bwd_flops(B, H, N, d, causal)


def test_headline_flops_value():
    # causal B=8 H=32 N=4096 d=128: 2 n^2 d per (b, h)
    assert bench.prefill_flops(8, 32, 4096, 128, True) == 1_099_511_627_776


def test_hstu_flops_over_jagged_lengths():
    from synthgen import workloads as W

    x = W.jagged_inputs(W.HSTU_JAGGED)
    c = W.HSTU_JAGGED
    assert bench.hstu_flops(x.lengths, c.H, c.d) == oracle.hstu_flops(x.lengths, c.H, c.d, True)
    assert bench.hstu_flops([3, 0, 5], 2, 4, False) == oracle.hstu_flops([3, 0, 5], 2, 4, False)


def test_decode_bytes_count_each_valid_cache_row_once():
    from oracle import cpp
    from synthgen import bf16_bits_to_f64 as f
    from synthgen import workloads as W

    c = W.Decode("bytes_pin", 3, 8, 2, 64, 128, 0.1, 1, 64, 14)
    x = W.decode_inputs(c, seqlens=[0, 5, 64])
    counts = {}
    cpp.decode(f(x.q), f(x.k), f(x.v), x.seqlens, c.scale, counts=counts)
    # the oracle reads each valid K and V row once per query head: d multiply-adds
    # per (head, row) and product; the bytes count each row once per kv head
    rows = counts["macs"] // (2 * c.d * (c.H // c.Hkv))
    assert rows == c.Hkv * int(np.sum(x.seqlens))
    expect = rows * c.d * 2 * 2 + 2 * c.B * c.H * c.d * 2 + c.B * c.H * 4 + c.B * 4
    assert bench.decode_bytes(x.seqlens, c.B, c.H, c.Hkv, c.d) == expect
