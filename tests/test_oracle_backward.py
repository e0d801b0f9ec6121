"""Pins of the fp64 backward oracle (``oracle.attention_backward``).

The gradient formulas are checked against things they do not share code with:
central finite differences of the forward oracle, torch autograd through a
plain fp64 softmax-attention graph, and invariants of the softmax Jacobian.
"""

import numpy as np
import pytest
import torch

import oracle


# run against both implementations: the C++ oracle and the numpy one
IMPLS = {"cpp": oracle.cpp, "numpy": oracle.numpy_ref}


@pytest.fixture(params=sorted(IMPLS))
def orc(request):
    return IMPLS[request.param]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(orc, q, k, v, r, scale, causal):
    o, _ = orc.attention_forward(q, k, v, scale, causal)
    return float((o * r).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(orc, causal):
    # loss = sum(O * R); its gradient wrt O is R, so dO = R
    B, H, Hkv, N, d = 1, 2, 1, 5, 3
    q, k, v = _rand((B, H, N, d), 1), _rand((B, Hkv, N, d), 2), _rand((B, Hkv, N, d), 3)
    r = _rand((B, H, N, d), 4)
    scale = 0.7
    dq, dk, dv = orc.attention_backward(q, k, v, r, scale, causal)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if x is t else t for t in (q, k, v)]
            args_m = [xm if x is t else t for t in (q, k, v)]
            num[idx] = (_loss(orc, *args_p, r, scale, causal) - _loss(orc, *args_m, r, scale, causal)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(orc, causal):
    B, H, Hkv, N, d = 2, 4, 2, 33, 16
    q, k, v = _rand((B, H, N, d), 11), _rand((B, Hkv, N, d), 12), _rand((B, Hkv, N, d), 13)
    do = _rand((B, H, N, d), 14)
    scale = d ** -0.5
    dq, dk, dv = orc.attention_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    kk = tk.repeat_interleave(H // Hkv, dim=1)
    vv = tv.repeat_interleave(H // Hkv, dim=1)
    s = scale * torch.matmul(tq, kk.transpose(-1, -2).contiguous())
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_gradients_sum_to_zero(orc, causal):
    # adding the same vector to every key shifts each score row by a constant,
    # which softmax ignores: the key gradients of a head sum to zero
    B, H, Hkv, N, d = 2, 4, 2, 17, 8
    q, k, v = _rand((B, H, N, d), 21), _rand((B, Hkv, N, d), 22), _rand((B, Hkv, N, d), 23)
    do = _rand((B, H, N, d), 24)
    _, dk, _ = orc.attention_backward(q, k, v, do, 0.3, causal)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)


def test_backward_constant_values_give_zero_score_gradients(orc):
    # every value row equal: O does not depend on P, so dQ = dK = 0 and
    # dV (summed over the key rows) is the column sum of dO
    B, H, Hkv, N, d = 1, 2, 2, 9, 4
    q, k = _rand((B, H, N, d), 31), _rand((B, Hkv, N, d), 32)
    v = np.broadcast_to(_rand((B, Hkv, 1, d), 33), (B, Hkv, N, d)).copy()
    do = _rand((B, H, N, d), 34)
    dq, dk, dv = orc.attention_backward(q, k, v, do, 0.5, False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def test_backward_single_key_passes_do_through(orc):
    # N = 1: P = 1, so dV = dO (summed over the group), dQ = dK = 0
    B, H, Hkv, N, d = 2, 4, 1, 1, 8
    q, k, v = _rand((B, H, N, d), 41), _rand((B, Hkv, N, d), 42), _rand((B, Hkv, N, d), 43)
    do = _rand((B, H, N, d), 44)
    dq, dk, dv = orc.attention_backward(q, k, v, do, 0.25, True)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv[:, 0], do.sum(axis=1), atol=1e-12)
