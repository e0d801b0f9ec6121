"""Negative and positive controls of the parity checker (CPU only).

The GPU parity tests accept an output when ``bf16_ok`` / ``lse_ok`` (in
``tests/_util.py``) accept it against the oracle.  With N(0,1) inputs the
outputs are small (|O| ~ 0.03 for prefill, ~0.01 for decode, <= 5e-3 for
HSTU), so the absolute bounds alone would accept an all-zero output.  These
tests plant plausible mistakes in the ORACLE, on the CPU, on inputs drawn
like the real workloads, and check that the checker rejects each one:

* an all-zero output;
* the causal flag flipped;
* V shifted by one row (an off-by-one in the value index);
* the key/value head map swapped (grouped-query attention);
* for HSTU, also the sequence offsets shifted by one token.

The positive control: the correct oracle output, rounded to bf16 as the GPU
writes it (and the LSE rounded to f32), passes.
"""

import math

import numpy as np
import pytest

import oracle
from synthgen import bf16_bits_to_f64, f32_to_bf16_bits
from synthgen import workloads as W
from tests._util import bf16_ok, lse_ok


def as_bf16(x):
    return bf16_bits_to_f64(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def rejected(got_o, ref_o, got_l=None, ref_l=None):
    ok_o, _ = bf16_ok(as_bf16(got_o), ref_o)
    ok_l = True
    if got_l is not None:
        ok_l, _ = lse_ok(np.asarray(got_l, np.float32).astype(np.float64), ref_l)
    return not (ok_o and ok_l)


PREFILL = [W.Dense("ctl_prefill_d64", 1, 4, 2, 2048, 64, 1.0 / 8.0, True, "bf16", 1001),
           W.Dense("ctl_prefill_d128", 1, 4, 2, 1024, 128, 1.0 / math.sqrt(128.0), True, "bf16", 1002),
           W.Dense("ctl_prefill_d128_nc", 1, 4, 2, 1024, 128, 1.0 / math.sqrt(128.0), False, "bf16", 1002)]


@pytest.fixture(scope="module", params=PREFILL, ids=lambda c: c.name)
def prefill_case(request):
    c = request.param
    x = W.dense_inputs(c)
    q, k, v = x.f64("q"), x.f64("k"), x.f64("v")
    O, L = oracle.attention_forward(q, k, v, c.scale, c.causal)
    return c, q, k, v, O, L


def test_prefill_correct_output_passes(prefill_case):
    c, q, k, v, O, L = prefill_case
    assert not rejected(O, O, L, L)


def test_prefill_rejects_zeros(prefill_case):
    c, q, k, v, O, L = prefill_case
    assert rejected(np.zeros_like(O), O)


def test_prefill_rejects_flipped_causal_flag(prefill_case):
    c, q, k, v, O, L = prefill_case
    O2, L2 = oracle.attention_forward(q, k, v, c.scale, not c.causal)
    assert rejected(O2, O, L2, L)
    assert rejected(O2, O)  # the output alone already gives it away


def test_prefill_rejects_values_shifted_by_one_row(prefill_case):
    c, q, k, v, O, L = prefill_case
    O2, L2 = oracle.attention_forward(q, k, np.roll(v, 1, axis=2), c.scale, c.causal)
    assert rejected(O2, O)


def test_prefill_rejects_swapped_kv_head_map(prefill_case):
    c, q, k, v, O, L = prefill_case
    O2, L2 = oracle.attention_forward(q, k[:, ::-1], v[:, ::-1], c.scale, c.causal)
    assert rejected(O2, O, L2, L)


def test_prefill_rejects_lse_in_base_two():
    c = PREFILL[1]
    x = W.dense_inputs(c)
    q, k, v = x.f64("q")[:, :1], x.f64("k")[:, :1], x.f64("v")[:, :1]
    _, L = oracle.attention_forward(q, k, v, c.scale, c.causal)
    S = c.scale * (q[0, 0] @ k[0, 0].T)
    if c.causal:
        S = np.where(np.tril(np.ones_like(S)) > 0, S, -np.inf)
    m = S.max(axis=1)
    wrong = m + np.log2(np.exp(L[0, 0] - m))  # log2 of the same sum of exponentials
    assert not lse_ok(wrong, L[0, 0])[0]
    assert lse_ok(L[0, 0].astype(np.float32).astype(np.float64), L[0, 0])[0]


DECODE = W.Decode("ctl_decode", 3, 8, 2, 32768, 128, 1.0 / math.sqrt(128.0), 16384, 32768, 1003)


@pytest.fixture(scope="module")
def decode_case():
    x = W.decode_inputs(DECODE)
    q, k, v = bf16_bits_to_f64(x.q), bf16_bits_to_f64(x.k), bf16_bits_to_f64(x.v)
    O, L = oracle.decode(q, k, v, x.seqlens, DECODE.scale)
    return x, q, k, v, O, L


def test_decode_correct_output_passes(decode_case):
    x, q, k, v, O, L = decode_case
    assert not rejected(O, O, L, L)


def test_decode_rejects_zeros(decode_case):
    x, q, k, v, O, L = decode_case
    assert rejected(np.zeros_like(O), O)


def test_decode_rejects_values_shifted_by_one_row(decode_case):
    x, q, k, v, O, L = decode_case
    v2 = np.roll(v, 1, axis=2)
    v2[:, :, 0] = v[:, :, 0]  # keep row 0 defined; every other row j reads v[j-1]
    O2, _ = oracle.decode(q, k, v2, x.seqlens, DECODE.scale)
    assert rejected(O2, O)


def test_decode_rejects_swapped_kv_head_map(decode_case):
    x, q, k, v, O, L = decode_case
    O2, L2 = oracle.decode(q, k[:, ::-1], v[:, ::-1], x.seqlens, DECODE.scale)
    assert rejected(O2, O, L2, L)


HSTU = W.Jagged("ctl_hstu", 4, 2, 64, 512, 4096, 1.0 / 8.0, 1.0 / 4096.0, True, 1004)


@pytest.fixture(scope="module")
def hstu_case():
    x = W.jagged_inputs(HSTU)
    q, k, v = bf16_bits_to_f64(x.q), bf16_bits_to_f64(x.k), bf16_bits_to_f64(x.v)
    O = oracle.hstu_jagged(q, k, v, x.offsets, HSTU.alpha, HSTU.inv_n, True)
    return x, q, k, v, O


def test_hstu_correct_output_passes(hstu_case):
    x, q, k, v, O = hstu_case
    assert not rejected(O, O)


def test_hstu_rejects_zeros(hstu_case):
    x, q, k, v, O = hstu_case
    assert np.abs(O).max() < 2e-2  # the absolute bound alone would accept zeros
    assert rejected(np.zeros_like(O), O)


def test_hstu_rejects_flipped_causal_flag(hstu_case):
    x, q, k, v, O = hstu_case
    assert rejected(oracle.hstu_jagged(q, k, v, x.offsets, HSTU.alpha, HSTU.inv_n, False), O)


def test_hstu_rejects_values_shifted_by_one_row(hstu_case):
    x, q, k, v, O = hstu_case
    assert rejected(oracle.hstu_jagged(q, k, np.roll(v, 1, axis=0), x.offsets, HSTU.alpha, HSTU.inv_n, True), O)


def test_hstu_rejects_offsets_shifted_by_one_token(hstu_case):
    x, q, k, v, O = hstu_case
    off = x.offsets.copy()
    off[1:-1] += 1  # every sequence boundary one token late
    assert rejected(oracle.hstu_jagged(q, k, v, off, HSTU.alpha, HSTU.inv_n, True), O)
