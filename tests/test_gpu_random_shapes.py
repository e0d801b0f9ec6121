"""Seeded random-shape parity sweep of every entry point against the fp64
oracle (prefill, decode contiguous and paged, jagged HSTU, backward, FP8
prefill): each case draws its own shape (batch, heads, group size, sequence
length, head dim, causal flag, scale; decode lengths including 0 and Lmax,
split counts, page sizes; jagged lengths including empty sequences) and is
compared on every output element.  The case parameters are in the test id and
the failure message.
"""

import math

import numpy as np
import pytest

import exact_attention_11_amd as fa
import oracle
from synthgen import TENSOR_K, TENSOR_Q, TENSOR_V, bf16_bits_to_f64, normal_bf16
from synthgen import workloads as W

from _util import assert_bf16, assert_lse, bf16_dev_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _prefill_case(i):
    r = np.random.default_rng(np.random.SeedSequence([7001, i]))
    d = int(r.choice([64, 128, 256]))
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.integers(1, 3))
    B = int(r.integers(1, 3))
    N = int(np.exp(r.uniform(0, math.log(600)))) if r.random() < 0.4 else int(r.integers(100, 601))
    causal = int(r.integers(0, 2))
    scale = float(1 / math.sqrt(d)) if r.random() < 0.5 else float(r.uniform(0.01, 0.3))
    return dict(B=B, H=G * Hkv, Hkv=Hkv, N=N, d=d, causal=causal, scale=scale, seed=7100 + i)


@pytest.mark.parametrize("i", range(96))
def test_random_prefill(i):
    _need_gpu()
    c = _prefill_case(i)
    B, H, Hkv, N, d = c["B"], c["H"], c["Hkv"], c["N"], c["d"]
    q = normal_bf16(c["seed"], TENSOR_Q, (B, H, N, d))
    k = normal_bf16(c["seed"], TENSOR_K, (B, Hkv, N, d))
    v = normal_bf16(c["seed"], TENSOR_V, (B, Hkv, N, d))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.attn_fwd(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), o, lse, B, H, Hkv, N, d, c["scale"], c["causal"])
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_forward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                            c["scale"], bool(c["causal"]))
    assert_bf16(bf16_dev_to_f64(o), O_ref, str(c))
    assert_lse(lse.cpu().numpy(), L_ref, str(c))


def _decode_case(i):
    r = np.random.default_rng(np.random.SeedSequence([7002, i]))
    G = int(r.choice([1, 2, 4, 8, 16, 32]))
    Hkv = int(r.integers(1, 3))
    B = int(r.integers(1, 6))
    Lmax = int(np.exp(r.uniform(0, math.log(1500)))) if r.random() < 0.3 else int(r.integers(200, 1501))
    lens = r.integers(0, Lmax + 1, size=B)
    lens[0] = Lmax
    if B > 2:
        lens[1] = 0
    splits = int(r.choice([0, 1, int(r.integers(2, 65))]))
    page = int(r.choice([16, 32, 64, 128, 512]))
    return dict(B=B, H=G * Hkv, Hkv=Hkv, Lmax=Lmax, lens=[int(x) for x in lens], splits=splits, page=page,
                seed=7200 + i)


@pytest.mark.parametrize("i", range(48))
def test_random_decode_contiguous_and_paged(i):
    _need_gpu()
    c = _decode_case(i)
    dc = W.Decode("random_decode", c["B"], c["H"], c["Hkv"], c["Lmax"], 128, 1 / math.sqrt(128), 0, c["Lmax"],
                  c["seed"])
    x = W.decode_inputs(dc, seqlens=c["lens"])
    q, k, v = to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)
    sl = to_dev(x.seqlens)
    # oracle: each sequence's rows [0, L_b) of the cache
    O_ref, L_ref = [], []
    for b in range(dc.B):
        n = int(x.seqlens[b])
        Ob, Lb = oracle.decode(bf16_bits_to_f64(x.q[b:b + 1]), bf16_bits_to_f64(x.k[b:b + 1, :, :n]),
                               bf16_bits_to_f64(x.v[b:b + 1, :, :n]), np.array([n]), dc.scale)
        O_ref.append(Ob[0])
        L_ref.append(Lb[0])
    O_ref, L_ref = np.stack(O_ref), np.stack(L_ref)
    # contiguous
    nbytes = fa.attn_decode_workspace_bytes(dc.B, dc.H, dc.d, c["splits"])
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o = torch.empty((dc.B, dc.H, dc.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((dc.B, dc.H), dtype=torch.float32, device="cuda")
    fa.attn_decode(q, k, v, sl, o, lse, dc.B, dc.H, dc.Hkv, dc.Lmax, dc.d, dc.scale, c["splits"], ws, nbytes)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(o)
    got_lse = lse.cpu().numpy()
    assert_bf16(got, O_ref, "contiguous " + str(c))
    assert_lse(got_lse, L_ref, "contiguous " + str(c))
    # paged (shuffled pages, NaN spare pages and tails), bitwise equal to contiguous
    px = W.paged_from_decode(x, c["page"], perm_seed=i)
    mp = px.block_table.shape[1]
    nbytes = fa.attn_decode_workspace_bytes(dc.B, dc.H, dc.d, c["splits"])
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    po = torch.empty_like(o)
    plse = torch.empty_like(lse)
    fa.attn_decode_paged(q, to_dev_bf16(px.k_pages), to_dev_bf16(px.v_pages), to_dev(px.block_table), sl, po, plse,
                         dc.B, dc.H, dc.Hkv, c["page"], mp, px.num_pages, dc.d, dc.scale, c["splits"], ws, nbytes)
    torch.cuda.synchronize()
    pgot = bf16_dev_to_f64(po)
    assert_bf16(pgot, O_ref, "paged " + str(c))
    assert_lse(plse.cpu().numpy(), L_ref, "paged " + str(c))
    if mp * c["page"] == dc.Lmax:  # same split boundaries: same arithmetic
        assert np.array_equal(pgot, got), "paged differs from contiguous " + str(c)


def _hstu_case(i):
    r = np.random.default_rng(np.random.SeedSequence([7003, i]))
    B = int(r.integers(1, 7))
    H = int(r.integers(1, 5))
    d = int(r.choice([64, 128]))
    lens = [int(x) for x in r.integers(0, 600, size=B)]
    if B > 1:
        lens[int(r.integers(1, B))] = 0
    lens[0] = max(lens[0], 1)
    causal = int(r.integers(0, 2))
    alpha = float(r.uniform(0.05, 0.5))
    return dict(B=B, H=H, d=d, lens=lens, causal=causal, alpha=alpha, seed=7300 + i)


@pytest.mark.parametrize("i", range(48))
def test_random_hstu(i):
    _need_gpu()
    c = _hstu_case(i)
    # 1/n keeps the outputs at the workloads' scale (|O| well below 1), where the
    # absolute bounds of the comparison are calibrated; the relative bounds apply too
    jc = W.Jagged("random_hstu", c["B"], c["H"], c["d"], 0, 600, c["alpha"], 1.0 / 512, bool(c["causal"]), c["seed"],
                  1.0)
    x = W.jagged_inputs(jc, lengths=c["lens"])
    T = int(x.offsets[-1])
    o = torch.full((max(T, 1), jc.H, jc.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    fa.attn_hstu_jagged(to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v), o, to_dev(x.offsets), jc.nseq, jc.H,
                        jc.d, max(x.max_seqlen, 1), jc.alpha, jc.inv_n, c["causal"])
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(o)
    for b in range(jc.nseq):
        s, e = int(x.offsets[b]), int(x.offsets[b + 1])
        if e == s:
            continue
        sub = np.array([0, e - s], dtype=np.int64)
        ref = oracle.hstu_jagged(bf16_bits_to_f64(x.q[s:e]), bf16_bits_to_f64(x.k[s:e]), bf16_bits_to_f64(x.v[s:e]),
                                 sub, jc.alpha, jc.inv_n, bool(c["causal"]))
        assert_bf16(got[s:e], ref, f"seq {b} " + str(c))


def _bwd_case(i):
    r = np.random.default_rng(np.random.SeedSequence([7004, i]))
    d = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4]))
    Hkv = int(r.integers(1, 3))
    B = int(r.integers(1, 3))
    N = int(r.integers(1, 12)) if r.random() < 0.3 else int(r.integers(60, 400))
    causal = int(r.integers(0, 2))
    scale = float(1 / math.sqrt(d)) if r.random() < 0.5 else float(r.uniform(0.02, 0.2))
    return dict(B=B, H=G * Hkv, Hkv=Hkv, N=N, d=d, causal=causal, scale=scale, seed=7400 + i)


@pytest.mark.parametrize("i", range(32))
def test_random_backward(i):
    _need_gpu()
    from synthgen import TENSOR_DO

    from _util import assert_grad

    c = _bwd_case(i)
    B, H, Hkv, N, d = c["B"], c["H"], c["Hkv"], c["N"], c["d"]
    q = normal_bf16(c["seed"], TENSOR_Q, (B, H, N, d))
    k = normal_bf16(c["seed"], TENSOR_K, (B, Hkv, N, d))
    v = normal_bf16(c["seed"], TENSOR_V, (B, Hkv, N, d))
    do = normal_bf16(c["seed"], TENSOR_DO, (B, H, N, d))
    tq, tk, tv, tdo = (to_dev_bf16(x) for x in (q, k, v, do))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    fa.attn_fwd(tq, tk, tv, o, lse, B, H, Hkv, N, d, c["scale"], c["causal"])
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
    nbytes = fa.attn_bwd_workspace_bytes(B, H, N)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    fa.attn_bwd(tq, tk, tv, o, lse, tdo, dq, dk, dv, B, H, Hkv, N, d, c["scale"], c["causal"], ws, nbytes)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                           bf16_bits_to_f64(do), c["scale"], bool(c["causal"]))
    assert_grad(bf16_dev_to_f64(dq), rq, "dQ " + str(c))
    assert_grad(bf16_dev_to_f64(dk), rk, "dK " + str(c))
    assert_grad(bf16_dev_to_f64(dv), rv, "dV " + str(c))


def _fp8_case(i):
    r = np.random.default_rng(np.random.SeedSequence([7005, i]))
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.integers(1, 3))
    B = int(r.integers(1, 3))
    N = int(r.integers(1, 12)) if r.random() < 0.3 else int(r.integers(60, 500))
    causal = int(r.integers(0, 2))
    return dict(B=B, H=G * Hkv, Hkv=Hkv, N=N, causal=causal, seed=7500 + i)


@pytest.mark.parametrize("i", range(32))
def test_random_fp8(i):
    _need_gpu()
    from _util import assert_fp8

    c = _fp8_case(i)
    dc = W.Dense("random_fp8", c["B"], c["H"], c["Hkv"], c["N"], 128, 1 / math.sqrt(128), bool(c["causal"]), "fp8",
                 c["seed"])
    x = W.fp8_dense_inputs(dc)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    o = torch.empty((dc.B, dc.H, dc.N, dc.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((dc.B, dc.H, dc.N), dtype=torch.float32, device="cuda")
    fa.attn_fwd_fp8(t(x.q), t(x.k), t(x.v), o, lse, t(x.descale_q), t(x.descale_k), t(x.descale_v), dc.B, dc.H,
                    dc.Hkv, dc.N, dc.d, dc.scale, int(dc.causal))
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_forward(x.f64("q"), x.f64("k"), x.f64("v"), dc.scale, bool(dc.causal))
    assert_fp8(bf16_dev_to_f64(o), O_ref, str(c))
    assert_lse(lse.cpu().numpy(), L_ref, str(c))
