"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every output element and span several tiles with ragged
tails.  The full-size workloads run in the launch configuration the benchmark
times and compare every output element, except the N = 32768 sequence (every
head on sampled rows).
"""

import math

import numpy as np
import pytest

import exact_attention_11_amd as fa
import oracle
from synthgen import TENSOR_K, TENSOR_Q, TENSOR_V, bf16_bits_to_f64, normal_bf16, normal_f32
from synthgen import workloads as W

from _util import (assert_bf16, assert_lse, bf16_dev_to_f64, f32_ok, lse_ok, sample_rows, to_dev,
                    to_dev_bf16)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_fwd(q_bits, k_bits, v_bits, B, H, Hkv, N, d, scale, causal, want_lse=True):
    q, k, v = to_dev_bf16(q_bits), to_dev_bf16(k_bits), to_dev_bf16(v_bits)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda") if want_lse else None
    fa.attn_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal)
    torch.cuda.synchronize()
    return o, lse


# --- f32 path ------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_tiny_f32_workload(causal):
    _need_gpu()
    c = W.TINY_F32
    x = W.dense_inputs(c)
    O_ref, L_ref = oracle.attention_forward(x.f64("q"), x.f64("k"), x.f64("v"), c.scale, causal)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H, c.N), dtype=torch.float32, device="cuda")
    fa.attn_fwd_f32(q, k, v, o, lse, c.B, c.H, c.Hkv, c.N, c.d, c.scale, int(causal))
    torch.cuda.synchronize()
    ok, r = f32_ok(o.cpu().numpy(), O_ref)
    assert ok, str(r)
    ok, r = lse_ok(lse.cpu().numpy(), L_ref)
    assert ok and r.max_abs <= 1e-5, str(r)


@pytest.mark.parametrize("N", [1, 63, 64, 65, 200])
def test_f32_ragged_and_gqa(N):
    _need_gpu()
    B, H, Hkv, d, scale = 2, 4, 2, 64, 0.125
    q = normal_f32(7, TENSOR_Q, (B, H, N, d))
    k = normal_f32(7, TENSOR_K, (B, Hkv, N, d))
    v = normal_f32(7, TENSOR_V, (B, Hkv, N, d))
    for causal in (0, 1):
        O_ref, L_ref = oracle.attention_forward(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                                scale, bool(causal))
        o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        fa.attn_fwd_f32(to_dev(q), to_dev(k), to_dev(v), o, lse, B, H, Hkv, N, d, scale, causal)
        torch.cuda.synchronize()
        ok, r = f32_ok(o.cpu().numpy(), O_ref)
        assert ok, f"causal={causal}: {r}"
        assert lse_ok(lse.cpu().numpy(), L_ref)[0]


# --- bf16 prefill, small shapes (every element) -------------------------------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 7, 64, 129, 255, 300])
@pytest.mark.parametrize("causal", [0, 1])
def test_bf16_small_every_element(d, N, causal):
    _need_gpu()
    B, H, Hkv = 2, 4, 2
    scale = 1.0 / math.sqrt(d)
    seed = 100 + N + d
    q = normal_bf16(seed, TENSOR_Q, (B, H, N, d))
    k = normal_bf16(seed, TENSOR_K, (B, Hkv, N, d))
    v = normal_bf16(seed, TENSOR_V, (B, Hkv, N, d))
    o, lse = run_fwd(q, k, v, B, H, Hkv, N, d, scale, causal)
    O_ref, L_ref = oracle.attention_forward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), scale,
                                            bool(causal))
    assert_bf16(bf16_dev_to_f64(o), O_ref, f"N={N} d={d} causal={causal}")
    assert_lse(lse.cpu().numpy(), L_ref, f"N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [0, 1])
def test_bf16_multi_query_one_kv_head(causal):
    # multi-query attention: every query head reads the single kv head
    _need_gpu()
    B, H, Hkv, N, d = 2, 8, 1, 150, 128
    scale = 1.0 / math.sqrt(d)
    q = normal_bf16(61, TENSOR_Q, (B, H, N, d))
    k = normal_bf16(61, TENSOR_K, (B, Hkv, N, d))
    v = normal_bf16(61, TENSOR_V, (B, Hkv, N, d))
    o, lse = run_fwd(q, k, v, B, H, Hkv, N, d, scale, causal)
    O_ref, L_ref = oracle.attention_forward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), scale,
                                            bool(causal))
    assert_bf16(bf16_dev_to_f64(o), O_ref, f"MQA causal={causal}")
    assert_lse(lse.cpu().numpy(), L_ref, f"MQA causal={causal}")


def test_decode_multi_query_32_heads():
    # 32 query heads on one kv head, the longest lengths of the decode workload
    _need_gpu()
    c = W.Decode("decode_mqa", 4, 32, 1, 4096, 128, 1 / math.sqrt(128), 1, 4096, 33)
    x = W.decode_inputs(c, seqlens=[4096, 1, 2500, 3333])
    o, lse = run_decode(x, 0)
    O_ref, L_ref = decode_ref(x)
    assert_bf16(o, O_ref, "MQA decode")
    assert_lse(lse, L_ref, "MQA decode")


@pytest.mark.parametrize("N", [1, 7, 33, 129, 300])
@pytest.mark.parametrize("causal", [0, 1])
def test_bf16_d256_every_element(N, causal):
    _need_gpu()
    B, H, Hkv, d = 2, 4, 2, 256
    scale = 1.0 / math.sqrt(d)
    q = normal_bf16(400 + N, TENSOR_Q, (B, H, N, d))
    k = normal_bf16(400 + N, TENSOR_K, (B, Hkv, N, d))
    v = normal_bf16(400 + N, TENSOR_V, (B, Hkv, N, d))
    o, lse = run_fwd(q, k, v, B, H, Hkv, N, d, scale, causal)
    O_ref, L_ref = oracle.attention_forward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), scale,
                                            bool(causal))
    assert_bf16(bf16_dev_to_f64(o), O_ref, f"d=256 N={N} causal={causal}")
    assert_lse(lse.cpu().numpy(), L_ref, f"d=256 N={N} causal={causal}")


@pytest.mark.timeout(600)
def test_bf16_d256_long_every_element():
    # B=2, H=16, N=4096, d=256 causal: every element
    _need_gpu()
    c = W.Dense("prefill_d256", 2, 16, 16, 4096, 256, 1.0 / 16.0, True, "bf16", 1005)
    for b in range(c.B):
        _check_batch(c, b)


def test_bf16_causal_row_zero_is_exactly_v0():
    _need_gpu()
    B, H, N, d = 1, 3, 200, 128
    q = normal_bf16(5, TENSOR_Q, (B, H, N, d))
    k = normal_bf16(5, TENSOR_K, (B, H, N, d))
    v = normal_bf16(5, TENSOR_V, (B, H, N, d))
    o, lse = run_fwd(q, k, v, B, H, H, N, d, 0.1, 1)
    got = o.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[:, :, 0], v[:, :, 0])
    s00 = 0.1 * np.einsum("bhd,bhd->bh", bf16_bits_to_f64(q[:, :, 0]), bf16_bits_to_f64(k[:, :, 0]))
    assert np.max(np.abs(lse.cpu().numpy()[:, :, 0] - s00)) < 1e-5


def test_bf16_zero_scale_is_running_mean():
    _need_gpu()
    B, H, N, d = 1, 2, 150, 64
    q = normal_bf16(6, TENSOR_Q, (B, H, N, d))
    k = normal_bf16(6, TENSOR_K, (B, H, N, d))
    v = normal_bf16(6, TENSOR_V, (B, H, N, d))
    for causal in (0, 1):
        o, lse = run_fwd(q, k, v, B, H, H, N, d, 0.0, causal)
        O_ref, L_ref = oracle.attention_forward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 0.0,
                                                bool(causal))
        assert_bf16(bf16_dev_to_f64(o), O_ref, f"scale=0 causal={causal}")
        assert_lse(lse.cpu().numpy(), L_ref)


def test_bf16_deterministic_and_lse_optional():
    _need_gpu()
    B, H, N, d = 1, 4, 333, 128
    q = normal_bf16(8, TENSOR_Q, (B, H, N, d))
    k = normal_bf16(8, TENSOR_K, (B, H, N, d))
    v = normal_bf16(8, TENSOR_V, (B, H, N, d))
    o1, l1 = run_fwd(q, k, v, B, H, H, N, d, 0.09, 1)
    o2, l2 = run_fwd(q, k, v, B, H, H, N, d, 0.09, 1)
    o3, _ = run_fwd(q, k, v, B, H, H, N, d, 0.09, 1, want_lse=False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_bf16_large_score_offset_no_overflow():
    """Scores around +-100 (far beyond exp range without the max shift)."""
    _need_gpu()
    B, H, N, d = 1, 2, 257, 128
    q = normal_bf16(9, TENSOR_Q, (B, H, N, d), 4.0)
    k = normal_bf16(9, TENSOR_K, (B, H, N, d), 4.0)
    v = normal_bf16(9, TENSOR_V, (B, H, N, d))
    for causal in (0, 1):
        o, lse = run_fwd(q, k, v, B, H, H, N, d, 1.0 / math.sqrt(d), causal)
        O_ref, L_ref = oracle.attention_forward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                                1.0 / math.sqrt(d), bool(causal))
        assert_bf16(bf16_dev_to_f64(o), O_ref, f"offset causal={causal}")
        assert_lse(lse.cpu().numpy(), L_ref)


# --- bf16 prefill, full-size workloads -------------------------------------------------
#
# Each workload runs once on the GPU (the launch configuration the benchmark
# times); its tests then compare one batch each against the oracle, so that
# no single test runs long.  Every element is compared, except for the
# N = 32768 sequence, whose oracle cost is 8.8e12 FLOP: there every head is
# compared on sampled rows (the first and last two query blocks, both rows
# around each 32-key tile boundary, every 61st row).

_FULL = {}


def _full_run(case):
    """Inputs (bf16 bits) and GPU outputs of one full-size workload; only the
    workload under test is kept in memory."""
    if case.name not in _FULL:
        _FULL.clear()
        x = W.dense_inputs(case)
        o, lse = run_fwd(x.q, x.k, x.v, case.B, case.H, case.Hkv, case.N, case.d, case.scale, int(case.causal))
        o_np = o.view(torch.int16).cpu().numpy().view(np.uint16)
        lse_np = lse.cpu().numpy()
        del o, lse
        assert np.isfinite(lse_np).all()
        _FULL[case.name] = (x, o_np, lse_np)
    return _FULL[case.name]


def _check_batch(case, b, heads=None, rows=None):
    """Compare batch b (all heads, or `heads`) on every row (or `rows`)."""
    x, o_np, lse_np = _full_run(case)
    heads = list(range(case.H)) if heads is None else list(heads)
    group = case.H // case.Hkv
    bs = slice(b, b + 1)
    q = x.f64("q", (bs, heads))
    k = x.f64("k", (bs, [h // group for h in heads]))  # one kv head per query head, in order
    v = x.f64("v", (bs, [h // group for h in heads]))
    O_ref, L_ref = oracle.attention_forward(q, k, v, case.scale, case.causal, rows=rows)
    rsel = slice(None) if rows is None else rows
    got = bf16_bits_to_f64(o_np[b][heads][:, rsel])
    what = f"{case.name} b={b} heads={heads[0]}..{heads[-1]}"
    assert_bf16(got, O_ref[0], what)
    assert_lse(lse_np[b][heads][:, rsel], L_ref[0], what)


@pytest.mark.timeout(600)
def test_full_prefill_d64_causal_every_element():
    _need_gpu()
    _check_batch(W.PREFILL_D64, 0)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case,b", [(c, b) for c in (W.PREFILL_D128_CAUSAL, W.PREFILL_D128_FULL) for b in range(8)],
                         ids=lambda v: v.name if isinstance(v, W.Dense) else f"b{v}")
def test_full_prefill_d128_every_element(case, b):
    _need_gpu()
    _check_batch(case, b)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("d,N", [(64, 1100), (128, 900)])
def test_prefill_causal_multi_round_ragged(d, N):
    """Causal grids too large to pair (B*H*ceil(nq/2) above the resident
    workgroups: 1024 for d = 64, 768 for d = 128) take one query block per
    workgroup, heaviest first; N is not a multiple of the 128-row block.
    Every element of every batch."""
    _need_gpu()
    case = W.Dense(f"prefill_multi_round_d{d}", 8, 32, 8, N, d, 1.0 / math.sqrt(d), True, "bf16", 1010 + d)
    for b in range(case.B):
        _check_batch(case, b)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("h0", [0, 8, 16, 24])
def test_full_prefill_long_causal_sampled_rows(h0):
    _need_gpu()
    _check_batch(W.PREFILL_LONG, 0, heads=range(h0, h0 + 8), rows=sample_rows(W.PREFILL_LONG.N))


# --- decode ----------------------------------------------------------------------------

def run_decode(x: W.DecodeInputs, splits: int):
    c = x.case
    q, k, v = to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)
    sl = to_dev(x.seqlens)
    o = torch.empty((c.B, c.H, c.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((c.B, c.H), dtype=torch.float32, device="cuda")
    nbytes = fa.attn_decode_workspace_bytes(c.B, c.H, c.d, splits)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    fa.attn_decode(q, k, v, sl, o, lse, c.B, c.H, c.Hkv, c.Lmax, c.d, c.scale, splits, ws, nbytes)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(o), lse.cpu().numpy()


def decode_ref(x: W.DecodeInputs, batches=None):
    c = x.case
    batches = range(c.B) if batches is None else batches
    O, L = [], []
    for b in batches:
        n = int(x.seqlens[b])
        kk = bf16_bits_to_f64(x.k[b:b + 1, :, :n])
        vv = bf16_bits_to_f64(x.v[b:b + 1, :, :n])
        Ob, Lb = oracle.decode(bf16_bits_to_f64(x.q[b:b + 1]), kk, vv, np.array([n]), c.scale)
        O.append(Ob[0])
        L.append(Lb[0])
    return np.stack(O), np.stack(L)


@pytest.mark.parametrize("splits", [0, 1, 3, 7, 64])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32])
def test_decode_small(splits, G):
    _need_gpu()
    Hkv = 2
    c = W.Decode("decode_small", 4, G * Hkv, Hkv, 700, 128, 1 / math.sqrt(128), 1, 700, 31)
    x = W.decode_inputs(c, seqlens=[1, 17, 513, 700])
    o, lse = run_decode(x, splits)
    O_ref, L_ref = decode_ref(x)
    assert_bf16(o, O_ref, f"G={G} splits={splits}")
    assert_lse(lse, L_ref, f"G={G} splits={splits}")


def test_decode_zero_length_sequence():
    _need_gpu()
    c = W.Decode("decode_empty", 2, 8, 2, 64, 128, 0.1, 1, 64, 32)
    x = W.decode_inputs(c, seqlens=[0, 40])
    o, lse = run_decode(x, 0)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    O_ref, L_ref = decode_ref(x, [1])
    assert_bf16(o[1:], O_ref)
    assert_lse(lse[1:], L_ref)


@pytest.mark.parametrize("splits", [0, 5])
def test_decode_every_sequence_empty(splits):
    """No key blocks at all: every work item exits at once and the combine
    alone writes O = 0 and LSE = -inf for every (sequence, head)."""
    _need_gpu()
    c = W.Decode("decode_all_empty", 3, 8, 2, 64, 128, 0.1, 1, 64, 37)
    x = W.decode_inputs(c, seqlens=[0, 0, 0])
    o, lse = run_decode(x, splits)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_decode_reused_workspace_with_random_contents():
    """The workspace needs no clearing: random bytes on entry, then calls with
    other split counts on the same buffer, each checked against the oracle;
    two calls with equal arguments agree bitwise."""
    _need_gpu()
    c = W.Decode("decode_reuse", 3, 16, 4, 900, 128, 1 / math.sqrt(128), 1, 900, 33)
    x = W.decode_inputs(c, seqlens=[5, 333, 900])
    q, k, v = to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)
    sl = to_dev(x.seqlens)
    nbytes = max(fa.attn_decode_workspace_bytes(c.B, c.H, c.d, s) for s in (1, 5, 13, 64))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen)
    O_ref, L_ref = decode_ref(x)
    prev = None
    for splits in (13, 13, 5, 64, 1, 13):
        o = torch.empty((c.B, c.H, c.d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((c.B, c.H), dtype=torch.float32, device="cuda")
        fa.attn_decode(q, k, v, sl, o, lse, c.B, c.H, c.Hkv, c.Lmax, c.d, c.scale, splits, ws, nbytes)
        torch.cuda.synchronize()
        got = bf16_dev_to_f64(o)
        assert_bf16(got, O_ref, f"splits={splits}")
        assert_lse(lse.cpu().numpy(), L_ref, f"splits={splits}")
        if splits == 13 and prev is not None:
            assert np.array_equal(got, prev), "equal calls differ"
        if splits == 13:
            prev = got


@pytest.mark.parametrize("splits", [0, 16, 64])
def test_full_decode_gqa(splits):
    _need_gpu()
    x = W.decode_inputs(W.DECODE_GQA)
    o, lse = run_decode(x, splits)
    O_ref, L_ref = decode_ref(x)
    assert_bf16(o, O_ref, f"decode splits={splits}")
    assert_lse(lse, L_ref, f"decode splits={splits}")


# --- jagged HSTU -------------------------------------------------------------------------

def run_hstu(x: W.JaggedInputs, causal: int):
    c = x.case
    T = int(x.offsets[-1])
    q, k, v = to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)
    off = to_dev(x.offsets)
    o = torch.full((T, c.H, c.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    fa.attn_hstu_jagged(q, k, v, o, off, len(x.lengths), c.H, c.d, x.max_seqlen, c.alpha, c.inv_n, causal)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(o)


def hstu_ref(x: W.JaggedInputs, causal: bool, seqs=None):
    c = x.case
    seqs = range(len(x.lengths)) if seqs is None else seqs
    out = {}
    for b in seqs:
        s, e = int(x.offsets[b]), int(x.offsets[b + 1])
        sub = np.array([0, e - s], dtype=np.int64)
        out[b] = oracle.hstu_jagged(bf16_bits_to_f64(x.q[s:e]), bf16_bits_to_f64(x.k[s:e]),
                                    bf16_bits_to_f64(x.v[s:e]), sub, c.alpha, c.inv_n, causal)
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_hstu_small_every_element(d, causal):
    _need_gpu()
    c = W.Jagged("hstu_small", 6, 3, d, 1, 300, 0.3, 1.0 / 64, bool(causal), 41, 1.0)
    x = W.jagged_inputs(c, lengths=[5, 0, 1, 129, 300, 64])
    o = run_hstu(x, causal)
    ref = hstu_ref(x, bool(causal))
    for b, r in ref.items():
        s, e = int(x.offsets[b]), int(x.offsets[b + 1])
        assert_bf16(o[s:e], r, f"seq {b} len {e - s}")


@pytest.mark.parametrize("B,H", [(70, 1), (1, 4), (65, 2), (64, 9)])
def test_hstu_d64_unbalanced_dispatch(B, H):
    """The d = 64 kernel deals (sequence, head) pairs to the XCDs by length
    only for 8 <= B*H <= 512 and B <= 64 (a wave ranks the sequences and one
    lane per pair of an XCD counts its blocks); more than 64 sequences, fewer
    than eight pairs or more than 512 take the plain pair-major mapping."""
    _need_gpu()
    rng = np.random.default_rng(B * 10 + H)
    lengths = [int(v) for v in rng.integers(0, 200, B)]
    lengths[B // 2] = 257
    c = W.Jagged("hstu_unbalanced", B, H, 64, 1, 257, 0.3, 1.0 / 64, True, 45, 1.0)
    x = W.jagged_inputs(c, lengths=lengths)
    o = run_hstu(x, 1)
    ref = hstu_ref(x, True)
    for b, r in ref.items():
        s, e = int(x.offsets[b]), int(x.offsets[b + 1])
        assert_bf16(o[s:e], r, f"seq {b} len {e - s}")


@pytest.mark.parametrize("B,H,zeros", [(64, 8, 9), (16, 32, 3), (9, 1, 8)])
def test_hstu_d64_balanced_dispatch_limits(B, H, zeros):
    """The balanced d = 64 mapping at its limits: 512 pairs (64 per XCD, one
    per lane of the list lookup) with 64 or 16 sequences, and 8 pairs with all
    sequences but one empty (every other workgroup finds no item)."""
    _need_gpu()
    rng = np.random.default_rng(B * 1000 + H)
    lengths = [int(v) for v in rng.integers(1, 160, B)]
    for i in rng.choice(B, size=zeros, replace=False):
        lengths[int(i)] = 0
    if max(lengths) == 0:
        lengths[0] = 97
    c = W.Jagged("hstu_balanced_limits", B, H, 64, 1, max(lengths), 0.3, 1.0 / 64, True, 46, 1.0)
    x = W.jagged_inputs(c, lengths=lengths)
    o = run_hstu(x, 1)
    ref = hstu_ref(x, True)
    for b, r in ref.items():
        s, e = int(x.offsets[b]), int(x.offsets[b + 1])
        assert_bf16(o[s:e], r, f"seq {b} len {e - s}")


def test_hstu_d128_multi_round():
    """d = 128 jagged HSTU whose grid is too large to pair (16 sequences x 4
    heads x 16 slots > 768 resident workgroups): one query block per
    workgroup, blocks past a sequence's end exit."""
    _need_gpu()
    lengths = [4096, 3000, 17, 0, 2049, 128, 1, 4000, 512, 640, 3333, 2, 1024, 4095, 100, 2500]
    c = W.Jagged("hstu_d128_multi_round", 16, 4, 128, 1, 4096, 0.125, 1.0 / 4096, True, 43, 0.5)
    x = W.jagged_inputs(c, lengths=lengths)
    o = run_hstu(x, 1)
    ref = hstu_ref(x, True, seqs=[0, 2, 3, 4, 6, 13])
    for b, r in ref.items():
        s0, e = int(x.offsets[b]), int(x.offsets[b + 1])
        assert_bf16(o[s0:e], r, f"seq {b} len {e - s0}")
    assert np.isfinite(o).all()


@pytest.mark.parametrize("causal", [0, 1])
def test_hstu_dense_padded_equals_jagged(causal):
    """Sequences zero-padded to a common length and run as equal-length
    sequences give the jagged result on every valid row (silu(0) = 0, so the
    zero keys and values contribute nothing), bitwise."""
    _need_gpu()
    c = W.Jagged("hstu_pad", 4, 2, 64, 1, 300, 0.3, 1.0 / 64, bool(causal), 42, 1.0)
    x = W.jagged_inputs(c, lengths=[300, 7, 0, 129])
    o = run_hstu(x, causal)
    Np = 300
    pad = {}
    for name in ("q", "k", "v"):
        src = getattr(x, name)
        dst = np.zeros((4 * Np, c.H, c.d), dtype=np.uint16)
        for b in range(4):
            s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
            dst[b * Np:b * Np + (s1 - s0)] = src[s0:s1]
        pad[name] = to_dev_bf16(dst)
    po = torch.empty((4 * Np, c.H, c.d), dtype=torch.bfloat16, device="cuda")
    off = torch.arange(0, 5 * Np, Np, dtype=torch.int32, device="cuda")
    fa.attn_hstu_jagged(pad["q"], pad["k"], pad["v"], po, off, 4, c.H, c.d, Np, c.alpha, c.inv_n, causal)
    torch.cuda.synchronize()
    got = po.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = o  # jagged result, f64 view of bf16
    for b in range(4):
        s0, s1 = int(x.offsets[b]), int(x.offsets[b + 1])
        assert np.array_equal(bf16_bits_to_f64(got[b * Np:b * Np + (s1 - s0)]), ref[s0:s1]), f"seq {b}"


@pytest.mark.timeout(600)
def test_full_hstu_jagged_every_sequence():
    _need_gpu()
    c = W.HSTU_JAGGED
    x = W.jagged_inputs(c)
    o = run_hstu(x, 1)
    assert np.isfinite(o).all()
    # the whole packed batch at once: every element of all 16 sequences
    ref = oracle.hstu_jagged(bf16_bits_to_f64(x.q), bf16_bits_to_f64(x.k), bf16_bits_to_f64(x.v), x.offsets,
                             c.alpha, c.inv_n, True)
    assert_bf16(o, ref, "all sequences")
    for b in range(len(x.lengths)):
        s, e = int(x.offsets[b]), int(x.offsets[b + 1])
        assert_bf16(o[s:e], ref[s:e], f"seq {b} len {e - s}")


def test_decode_clamps_lengths_to_the_cache():
    """seqlens_k is read only on the device and clamped to [0, Lmax]: a length
    past the cache gives the full-cache result, a negative one the empty
    result (O = 0, LSE = -inf), and nothing outside the cache is read."""
    _need_gpu()
    c = W.Decode("decode_clamp", 4, 8, 2, 700, 128, 1 / math.sqrt(128), 1, 700, 34)
    x = W.decode_inputs(c, seqlens=[700, 0, 0, 700])
    x.seqlens[:] = [700 + 500, -7, 0, 700]
    o, lse = run_decode(x, 0)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(o[2] == 0) and np.all(np.isneginf(lse[2]))
    x.seqlens[:] = [700, 0, 0, 700]
    O_ref, L_ref = decode_ref(x, [0, 3])
    assert_bf16(o[[0, 3]], O_ref)
    assert_lse(lse[[0, 3]], L_ref)


@pytest.mark.parametrize("splits", [1, 16])
def test_decode_partition_many_short_sequences(splits):
    """The work partition over sequence ends: 70 sequences (two groups of 64 in
    the kernels' prefix sums) of 0..96 keys.  With 1 split the 70 work items
    hold one or two blocks each and most cross a sequence end; with 16 there
    are more items than blocks, so only one item per block runs."""
    _need_gpu()
    B = 70
    c = W.Decode("decode_short", B, 8, 2, 96, 128, 1 / math.sqrt(128), 1, 96, 35)
    x = W.decode_inputs(c, seqlens=[(7 * b) % 97 for b in range(B)])
    o, lse = run_decode(x, splits)
    empty = x.seqlens == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    keep = np.flatnonzero(~empty)
    O_ref, L_ref = decode_ref(x, keep)
    assert_bf16(o[keep], O_ref, f"splits={splits}")
    assert_lse(lse[keep], L_ref, f"splits={splits}")


def test_decode_partition_one_long_sequence():
    """One sequence holds nearly all the blocks, so it is spread over ~126 of
    the 128 work items and the combine merges more than 64 partials; the other
    sequences are empty or a single block."""
    _need_gpu()
    c = W.Decode("decode_skew", 8, 16, 2, 9000, 128, 1 / math.sqrt(128), 1, 9000, 36)
    x = W.decode_inputs(c, seqlens=[9000, 0, 5, 0, 0, 32, 0, 1])
    o, lse = run_decode(x, 16)
    empty = x.seqlens == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    keep = np.flatnonzero(~empty)
    O_ref, L_ref = decode_ref(x, keep)
    assert_bf16(o[keep], O_ref)
    assert_lse(lse[keep], L_ref)


@pytest.mark.parametrize("causal", [0, 1])
def test_hstu_rows_past_max_seqlen_are_not_computed(causal):
    """A sequence longer than max_seqlen (a violated precondition) is cut to
    its first max_seqlen rows and keys: those rows match the oracle on the cut
    sequence, the rows past it are left as they were (NaN here), and nothing
    is read outside the sequence."""
    _need_gpu()
    c = W.Jagged("hstu_clamp", 3, 2, 64, 1, 300, 0.25, 1.0 / 64, bool(causal), 44, 1.0)
    x = W.jagged_inputs(c, lengths=[300, 50, 130])
    T = int(x.offsets[-1])
    q, k, v = to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)
    off = to_dev(x.offsets)
    o = torch.full((T, c.H, c.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    fa.attn_hstu_jagged(q, k, v, o, off, 3, c.H, c.d, 200, c.alpha, c.inv_n, causal)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(o)
    for b, keep in ((0, 200), (1, 50), (2, 130)):
        s = int(x.offsets[b])
        sub = np.array([0, keep], dtype=np.int64)
        ref = oracle.hstu_jagged(bf16_bits_to_f64(x.q[s:s + keep]), bf16_bits_to_f64(x.k[s:s + keep]),
                                 bf16_bits_to_f64(x.v[s:s + keep]), sub, c.alpha, c.inv_n, bool(causal))
        assert_bf16(got[s:s + keep], ref, f"seq {b}")
    assert np.isnan(got[200:300]).all()
