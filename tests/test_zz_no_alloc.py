"""attn_decode_noalloc -- the decode entry point for callers that cannot
allocate -- against attn_decode with a caller-supplied workspace, through the
C ABI, and against the oracle.

Two calls in a row on the static scratch array, the second with a smaller
input (so it runs over the first call's leftover partials), then the first
shape again at another split count.  The same kernels run in both entry
points, so the outputs must be bitwise equal; both must also meet the parity
bar against the oracle.
"""

import math

import numpy as np
import pytest

import exact_attention_11_amd as fa
import oracle
from synthgen import bf16_bits_to_f64
from synthgen import workloads as W

from _util import assert_bf16, assert_lse, bf16_dev_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(x, splits, noalloc):
    c = x.case
    q, k, v = to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)
    sl = to_dev(x.seqlens)
    o = torch.full((c.B, c.H, c.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c.B, c.H), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        fa.attn_decode_noalloc(q, k, v, sl, o, lse, c.B, c.H, c.Hkv, c.Lmax, c.d, c.scale, splits)
    else:
        nbytes = fa.attn_decode_workspace_bytes(c.B, c.H, c.d, splits)
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
        fa.attn_decode(q, k, v, sl, o, lse, c.B, c.H, c.Hkv, c.Lmax, c.d, c.scale, splits, ws, nbytes)
    torch.cuda.synchronize()
    return o.view(torch.int16).cpu().numpy(), lse.cpu().numpy()


def _ref(x):
    c = x.case
    return oracle.decode(bf16_bits_to_f64(x.q), bf16_bits_to_f64(x.k), bf16_bits_to_f64(x.v), x.seqlens, c.scale)


def test_noalloc_decode_matches_workspace_decode():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    big = W.decode_inputs(W.DECODE_GQA)
    small = W.decode_inputs(W.Decode("noalloc_small", 3, 8, 2, 700, 128, 1 / math.sqrt(128), 1, 700, 51),
                            seqlens=[1, 300, 700])
    for x, splits in ((big, 0), (small, 5), (big, 16)):
        c = x.case
        print(f"noalloc decode B={c.B} H={c.H} Hkv={c.Hkv} Lmax={c.Lmax} splits={splits}", flush=True)
        o_ws, l_ws = _run(x, splits, noalloc=False)
        o_na, l_na = _run(x, splits, noalloc=True)
        assert np.array_equal(o_na, o_ws), f"O differs from attn_decode (splits={splits})"
        assert np.array_equal(l_na, l_ws), f"LSE differs from attn_decode (splits={splits})"
        O_ref, L_ref = _ref(x)
        assert_bf16(bf16_bits_to_f64(o_na.view(np.uint16)), O_ref, f"{c.name} splits={splits}")
        assert_lse(l_na, L_ref, f"{c.name} splits={splits}")
