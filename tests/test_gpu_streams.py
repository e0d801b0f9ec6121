"""Calls on two streams at once: the library keeps no shared mutable state, so
work queued on two non-default streams without synchronisation in between must
give, call for call, exactly the bytes the same calls give one at a time on
the default stream (every kernel here is deterministic), and the prefill still
matches the oracle on sampled rows.
"""

import math

import numpy as np
import pytest

import exact_attention_11_amd as fa
import oracle
from synthgen import bf16_bits_to_f64
from synthgen import workloads as W

from _util import assert_bf16, assert_lse, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_two_streams_match_serial_calls_bitwise():
    _need_gpu()
    # prefill: causal, GQA, ragged tail, a grid of several rounds of workgroups
    pc = W.Dense("streams_prefill", 4, 16, 4, 1500, 128, 1 / math.sqrt(128), True, "bf16", 71)
    px = W.dense_inputs(pc)
    pq, pk, pv = to_dev_bf16(px.q), to_dev_bf16(px.k), to_dev_bf16(px.v)
    # decode: GQA with different history lengths
    dc = W.Decode("streams_decode", 4, 16, 4, 3000, 128, 1 / math.sqrt(128), 1, 3000, 72)
    dx = W.decode_inputs(dc, seqlens=[3000, 1, 1777, 640])
    dq, dk, dv, dsl = to_dev_bf16(dx.q), to_dev_bf16(dx.k), to_dev_bf16(dx.v), to_dev(dx.seqlens)
    # jagged HSTU
    jc = W.Jagged("streams_hstu", 5, 4, 64, 1, 1200, 0.125, 1.0 / 1024, True, 73)
    jx = W.jagged_inputs(jc, lengths=[1200, 3, 0, 700, 511])
    T = int(jx.offsets[-1])
    jq, jk, jv, joff = to_dev_bf16(jx.q), to_dev_bf16(jx.k), to_dev_bf16(jx.v), to_dev(jx.offsets)

    def outputs():
        return {
            "o": torch.empty((pc.B, pc.H, pc.N, pc.d), dtype=torch.bfloat16, device="cuda"),
            "lse": torch.empty((pc.B, pc.H, pc.N), dtype=torch.float32, device="cuda"),
            "do": torch.empty((dc.B, dc.H, dc.d), dtype=torch.bfloat16, device="cuda"),
            "dlse": torch.empty((dc.B, dc.H), dtype=torch.float32, device="cuda"),
            "ho": torch.empty((T, jc.H, jc.d), dtype=torch.bfloat16, device="cuda"),
        }

    wsb = fa.attn_decode_workspace_bytes(dc.B, dc.H, dc.d, 0)

    def prefill(out, stream=None):
        fa.attn_fwd(pq, pk, pv, out["o"], out["lse"], pc.B, pc.H, pc.Hkv, pc.N, pc.d, pc.scale, 1, stream)

    def decode(out, ws, stream=None):
        fa.attn_decode(dq, dk, dv, dsl, out["do"], out["dlse"], dc.B, dc.H, dc.Hkv, dc.Lmax, dc.d, dc.scale, 0,
                       ws, wsb, stream)

    def hstu(out, stream=None):
        fa.attn_hstu_jagged(jq, jk, jv, out["ho"], joff, len(jx.lengths), jc.H, jc.d, jx.max_seqlen, jc.alpha,
                            jc.inv_n, 1, stream)

    # one at a time on the default stream
    ref = outputs()
    ws0 = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    prefill(ref)
    decode(ref, ws0)
    hstu(ref)
    torch.cuda.synchronize()

    # interleaved on two streams (default priority), each with its own outputs
    # and decode workspace, three rounds queued before any synchronisation
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    wsa = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    wsb_ = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    rounds = []
    for _ in range(3):
        oa, ob = outputs(), outputs()
        prefill(oa, sa)
        decode(ob, wsb_, sb)
        hstu(ob, sb)
        decode(oa, wsa, sa)
        prefill(ob, sb)
        hstu(oa, sa)
        rounds.append((oa, ob))
    torch.cuda.synchronize()

    for i, (oa, ob) in enumerate(rounds):
        for name in ("o", "lse", "do", "dlse", "ho"):
            for tag, got in (("a", oa[name]), ("b", ob[name])):
                assert torch.equal(got.view(torch.uint8) if got.dtype == torch.bfloat16 else got,
                                   ref[name].view(torch.uint8) if got.dtype == torch.bfloat16 else ref[name]), \
                    f"round {i} stream {tag}: {name} differs from the serial call"

    # and the serial prefill is right: rows of two heads against the oracle
    rows = np.array([0, 1, 127, 128, 700, 1023, 1024, 1499])
    o = ref["o"].float().cpu().numpy()
    lse = ref["lse"].cpu().numpy()
    for b, h in ((0, 0), (3, 13)):
        g = h // (pc.H // pc.Hkv)
        O_ref, L_ref = oracle.attention_forward(bf16_bits_to_f64(px.q[b:b + 1, h:h + 1]),
                                                bf16_bits_to_f64(px.k[b:b + 1, g:g + 1]),
                                                bf16_bits_to_f64(px.v[b:b + 1, g:g + 1]), pc.scale, True, rows=rows)
        assert_bf16(o[b, h, rows], O_ref[0, 0], f"prefill b={b} h={h}")
        assert_lse(lse[b, h, rows], L_ref[0, 0], f"prefill b={b} h={h}")
