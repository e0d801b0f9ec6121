"""Parity of the FP8 prefill (``attn_fwd_fp8`` through the C ABI) against the
fp64 oracle evaluated on the dequantised inputs (fp8 value * descale), with
the E4M3 tolerance of ``tests/_util.py``."""

import math

import numpy as np
import pytest

import exact_attention_11_amd as fa
import oracle
from synthgen import bf16_bits_to_f64
from synthgen import workloads as W

from _util import assert_fp8, assert_lse

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_fp8(x: W.Fp8DenseInputs):
    c = x.case
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    o = torch.empty((c.B, c.H, c.N, c.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((c.B, c.H, c.N), dtype=torch.float32, device="cuda")
    fa.attn_fwd_fp8(t(x.q), t(x.k), t(x.v), o, lse, t(x.descale_q), t(x.descale_k), t(x.descale_v), c.B, c.H, c.Hkv,
                    c.N, c.d, c.scale, int(c.causal))
    torch.cuda.synchronize()
    return bf16_bits_to_f64(o.view(torch.int16).cpu().numpy().view(np.uint16)), lse.cpu().numpy()


@pytest.mark.parametrize("N", [1, 7, 64, 129, 300])
@pytest.mark.parametrize("causal", [0, 1])
def test_fp8_small_every_element(N, causal):
    _need_gpu()
    c = W.Dense("fp8_small", 2, 4, 2, N, 128, 1 / math.sqrt(128), bool(causal), "fp8", 500 + N)
    x = W.fp8_dense_inputs(c)
    o, lse = run_fp8(x)
    O_ref, L_ref = oracle.attention_forward(x.f64("q"), x.f64("k"), x.f64("v"), c.scale, bool(causal))
    assert_fp8(o, O_ref, f"N={N} causal={causal}")
    assert_lse(lse, L_ref, f"N={N} causal={causal}")


def test_fp8_per_head_descales_are_applied():
    # wide spread of descales between heads (sigma 0.25 .. 4 per head, one draw per head)
    _need_gpu()
    c = W.Dense("fp8_desc", 1, 4, 4, 200, 128, 1 / math.sqrt(128), True, "fp8", 77)
    x = W.fp8_dense_inputs(c)
    f = np.array([0.25, 1.0, 2.0, 4.0], dtype=np.float32)[None, :]
    x.descale_q = x.descale_q * f
    x.descale_v = x.descale_v / f
    o, lse = run_fp8(x)
    O_ref, L_ref = oracle.attention_forward(x.f64("q"), x.f64("k"), x.f64("v"), c.scale, True)
    assert_fp8(o, O_ref, "per-head descales")
    assert_lse(lse, L_ref, "per-head descales")


_FP8_FULL = {}


def _fp8_full():
    """Inputs and GPU outputs of the full-size FP8 workload, run once."""
    if not _FP8_FULL:
        x = W.fp8_dense_inputs(W.PREFILL_FP8)
        o, lse = run_fp8(x)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        _FP8_FULL["run"] = (x, o, lse)
    return _FP8_FULL["run"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("b", range(8))
def test_fp8_full_size_every_element(b):
    """B=8, H=32, N=4096, d=128 causal in FP8: every element of batch b."""
    _need_gpu()
    c = W.PREFILL_FP8
    x, o, lse = _fp8_full()
    idx = (slice(b, b + 1),)
    O_ref, L_ref = oracle.attention_forward(x.f64("q", idx), x.f64("k", idx), x.f64("v", idx), c.scale, True)
    assert_fp8(o[b], O_ref[0], f"b={b}")
    assert_lse(lse[b], L_ref[0], f"b={b}")
