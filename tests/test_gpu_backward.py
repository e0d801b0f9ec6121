"""Parity of the backward pass (``attn_bwd`` through the C ABI) against the
fp64 oracle's gradients.

The forward output and LSE that the backward consumes come from ``attn_fwd``
on the GPU (the product path's own data flow); the oracle computes the
gradients from q, k, v and dO alone.  Small cases compare every element over
several tiles with ragged tails; the full-size case compares every element
of two whole batches.
"""

import math

import numpy as np
import pytest

import exact_attention_11_amd as fa
import oracle
from synthgen import TENSOR_DO, TENSOR_K, TENSOR_Q, TENSOR_V, bf16_bits_to_f64, normal_bf16
from synthgen import workloads as W

from _util import assert_grad, bf16_dev_to_f64, to_dev_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_bwd(q_bits, k_bits, v_bits, do_bits, B, H, Hkv, N, d, scale, causal):
    q, k, v, do = (to_dev_bf16(x) for x in (q_bits, k_bits, v_bits, do_bits))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.attn_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    nbytes = fa.attn_bwd_workspace_bytes(B, H, N)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    fa.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, B, H, Hkv, N, d, scale, causal, ws, nbytes)
    torch.cuda.synchronize()
    return dq, dk, dv


def _inputs(seed, B, H, Hkv, N, d, sigma=1.0):
    return (normal_bf16(seed, TENSOR_Q, (B, H, N, d), sigma), normal_bf16(seed, TENSOR_K, (B, Hkv, N, d), sigma),
            normal_bf16(seed, TENSOR_V, (B, Hkv, N, d)), normal_bf16(seed, TENSOR_DO, (B, H, N, d)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 64, 129, 200])
@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_small_every_element(d, N, causal):
    _need_gpu()
    B, H, Hkv = 2, 4, 2
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = _inputs(300 + N + d, B, H, Hkv, N, d)
    dq, dk, dv = run_bwd(q, k, v, do, B, H, Hkv, N, d, scale, causal)
    rq, rk, rv = oracle.attention_backward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                           bf16_bits_to_f64(do), scale, bool(causal))
    tag = f"N={N} d={d} causal={causal}"
    assert_grad(bf16_dev_to_f64(dq), rq, "dQ " + tag)
    assert_grad(bf16_dev_to_f64(dk), rk, "dK " + tag)
    assert_grad(bf16_dev_to_f64(dv), rv, "dV " + tag)


@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_gqa_group_of_four_and_wide_scores(causal):
    # four query heads per kv-head (gradients summed over the group) and
    # larger scores (sigma 2 on q and k)
    _need_gpu()
    B, H, Hkv, N, d = 1, 8, 2, 190, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = _inputs(77, B, H, Hkv, N, d, sigma=2.0)
    dq, dk, dv = run_bwd(q, k, v, do, B, H, Hkv, N, d, scale, causal)
    rq, rk, rv = oracle.attention_backward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                           bf16_bits_to_f64(do), scale, bool(causal))
    assert_grad(bf16_dev_to_f64(dq), rq, "dQ")
    assert_grad(bf16_dev_to_f64(dk), rk, "dK")
    assert_grad(bf16_dev_to_f64(dv), rv, "dV")


def test_bwd_multi_query_one_kv_head():
    # every query head reads the single kv head: dK and dV sum over all eight
    _need_gpu()
    B, H, Hkv, N, d = 1, 8, 1, 130, 64
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = _inputs(79, B, H, Hkv, N, d)
    dq, dk, dv = run_bwd(q, k, v, do, B, H, Hkv, N, d, scale, 1)
    rq, rk, rv = oracle.attention_backward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                           bf16_bits_to_f64(do), scale, True)
    assert_grad(bf16_dev_to_f64(dq), rq, "dQ")
    assert_grad(bf16_dev_to_f64(dk), rk, "dK")
    assert_grad(bf16_dev_to_f64(dv), rv, "dV")


def test_bwd_deterministic():
    _need_gpu()
    B, H, Hkv, N, d = 1, 4, 1, 257, 64
    q, k, v, do = _inputs(78, B, H, Hkv, N, d)
    a = run_bwd(q, k, v, do, B, H, Hkv, N, d, 0.125, 1)
    b = run_bwd(q, k, v, do, B, H, Hkv, N, d, 0.125, 1)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.timeout(600)
def test_bwd_full_size_causal_two_batches():
    """B=8, H=32, N=4096, d=128 causal (the prefill benchmark shape), in the
    launch configuration the benchmark times: every element of dQ, dK and dV
    of batches 0 and 7 (all 32 heads of each)."""
    _need_gpu()
    c = W.PREFILL_D128_CAUSAL
    x = W.dense_inputs(c)
    do = normal_bf16(c.seed, TENSOR_DO, (c.B, c.H, c.N, c.d))
    dq, dk, dv = run_bwd(x.q, x.k, x.v, do, c.B, c.H, c.Hkv, c.N, c.d, c.scale, 1)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    for b in (0, 7):
        bs = slice(b, b + 1)
        rq, rk, rv = oracle.attention_backward(x.f64("q", (bs,)), x.f64("k", (bs,)), x.f64("v", (bs,)),
                                               bf16_bits_to_f64(do[bs]), c.scale, True)
        assert_grad(bf16_dev_to_f64(dq[b]), rq[0], f"dQ b={b}")
        assert_grad(bf16_dev_to_f64(dk[b]), rk[0], f"dK b={b}")
        assert_grad(bf16_dev_to_f64(dv[b]), rv[0], f"dV b={b}")
