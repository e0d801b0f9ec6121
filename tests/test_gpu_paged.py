"""Parity of the paged-cache decode (``attn_decode_paged`` through the C ABI)
against the fp64 oracle, and against the contiguous decode on the same data.

The pages hold the same cache as the contiguous tests, scattered in a seeded
random physical order; spare pages and rows past each sequence's length are
NaN, so any read outside the valid rows would show in the output.
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


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_paged(px: W.PagedDecodeInputs, splits: int):
    x = px.base
    c = x.case
    mp = px.block_table.shape[1]
    q, kp, vp = to_dev_bf16(x.q), to_dev_bf16(px.k_pages), to_dev_bf16(px.v_pages)
    table, sl = to_dev(px.block_table), to_dev(x.seqlens)
    o = torch.empty((c.B, c.H, c.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((c.B, c.H), dtype=torch.float32, device="cuda")
    nbytes = fa.attn_decode_workspace_bytes(c.B, c.H, c.d, splits)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    fa.attn_decode_paged(q, kp, vp, table, sl, o, lse, c.B, c.H, c.Hkv, px.page_size, mp, px.num_pages, c.d,
                         c.scale, splits, ws, nbytes)
    torch.cuda.synchronize()
    return o, lse


def run_contiguous(x: W.DecodeInputs, splits: int, Lmax: int):
    c = x.case
    q, k, v = to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)
    o = torch.empty((c.B, c.H, c.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((c.B, c.H), dtype=torch.float32, device="cuda")
    nbytes = fa.attn_decode_workspace_bytes(c.B, c.H, c.d, splits)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    fa.attn_decode(q, k, v, to_dev(x.seqlens), o, lse, c.B, c.H, c.Hkv, c.Lmax, c.d, c.scale, splits, ws, nbytes)
    torch.cuda.synchronize()
    return o, lse


def paged_ref(px: W.PagedDecodeInputs):
    x = px.base
    f = bf16_bits_to_f64
    return oracle.decode_paged(f(x.q), f(px.k_pages), f(px.v_pages), px.block_table, x.seqlens, x.case.scale)


@pytest.mark.parametrize("P", [16, 32, 64, 256])
@pytest.mark.parametrize("G", [1, 4, 16, 32])
@pytest.mark.parametrize("splits", [0, 1, 3, 7])
def test_paged_small_every_element(P, G, splits):
    _need_gpu()
    Hkv = 2
    c = W.Decode("paged_small", 5, G * Hkv, Hkv, 700, 128, 1 / math.sqrt(128), 1, 700, 51)
    x = W.decode_inputs(c, seqlens=[1, 17, 0, 513, 700])
    px = W.paged_from_decode(x, P, perm_seed=G * 100 + splits)
    o, lse = run_paged(px, splits)
    O_ref, L_ref = paged_ref(px)
    o64, l64 = bf16_dev_to_f64(o), lse.cpu().numpy()
    tag = f"P={P} G={G} splits={splits}"
    assert np.all(o64[2] == 0) and np.all(np.isneginf(l64[2])), tag
    keep = [0, 1, 3, 4]
    assert_bf16(o64[keep], O_ref[keep], tag)
    assert_lse(l64[keep], L_ref[keep], tag)


@pytest.mark.parametrize("P", [16, 64])
def test_paged_matches_contiguous_bitwise(P):
    # the same rows in the same order: the paged kernel differs only in where
    # it reads them from
    _need_gpu()
    c = W.Decode("paged_vs_contig", 3, 16, 4, 1024, 128, 1 / math.sqrt(128), 1, 1024, 52)
    x = W.decode_inputs(c, seqlens=[1000, 1024, 33])
    px = W.paged_from_decode(x, P)
    o1, l1 = run_paged(px, 8)
    o2, l2 = run_contiguous(x, 8, c.Lmax)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("P", [16, 64])
def test_full_paged_decode_gqa(P):
    """The decode workload (B=16, H=32, Hkv=8, L_b in [16384, 32768]) in pages
    of P rows, every output compared."""
    _need_gpu()
    px = W.paged_from_decode(W.decode_inputs(W.DECODE_GQA), P)
    o, lse = run_paged(px, 0)
    O_ref, L_ref = paged_ref(px)
    assert_bf16(bf16_dev_to_f64(o), O_ref, f"paged P={P}")
    assert_lse(lse.cpu().numpy(), L_ref, f"paged P={P}")


def test_paged_clamps_table_entries_and_lengths():
    """Block-table entries are clamped to [0, num_pages) and lengths to
    [0, max_pages_per_seq * page_size] on the device: an entry past the pool
    reads the pool's last page, a negative one page 0, and a length past the
    table the whole table."""
    _need_gpu()
    P = 64
    c = W.Decode("paged_clamp", 3, 8, 2, 704, 128, 1 / math.sqrt(128), 1, 704, 52)
    x = W.decode_inputs(c, seqlens=[704, 300, 704])
    px = W.paged_from_decode(x, P, spare_pages=0, perm_seed=9)
    O_ref, L_ref = paged_ref(px)
    last = px.num_pages - 1
    table = px.block_table.copy()
    ib, ip = np.argwhere(table == last)[0]
    jb, jp = np.argwhere(table == 0)[0]
    table[ib, ip] = last + 1000
    table[jb, jp] = -3
    x.seqlens[:] = [704 + 77, 300, 704 + 5000]
    bad = W.PagedDecodeInputs(x, P, px.k_pages, px.v_pages, table, px.num_pages)
    o, lse = run_paged(bad, 0)
    assert_bf16(bf16_dev_to_f64(o), O_ref, "clamped table and lengths")
    assert_lse(lse.cpu().numpy(), L_ref, "clamped table and lengths")


def test_paged_auto_splits_with_a_long_page_table():
    """Automatic split count with 128 (sequence, kv-head) pairs and a table of
    12,800 pages of 16 keys (Lmax = 204,800): the count is raised until no
    work item can span more than 2047 pages, so the call is accepted, and the
    short sequences still match the oracle.  Table entries past each
    sequence's pages are 0 and never read for keys."""
    _need_gpu()
    B, P, wide = 128, 16, 12800
    c = W.Decode("paged_wide_table", B, 1, 1, 96, 128, 1 / math.sqrt(128), 1, 96, 55)
    x = W.decode_inputs(c, seqlens=[(5 * b) % 97 for b in range(B)])
    px = W.paged_from_decode(x, P, perm_seed=55)
    table = np.zeros((B, wide), dtype=np.int32)
    table[:, :px.block_table.shape[1]] = px.block_table
    q, kp, vp = to_dev_bf16(x.q), to_dev_bf16(px.k_pages), to_dev_bf16(px.v_pages)
    o = torch.empty((B, 1, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1), dtype=torch.float32, device="cuda")
    nbytes = fa.attn_decode_workspace_bytes(B, 1, 128, 0)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    fa.attn_decode_paged(q, kp, vp, to_dev(table), to_dev(x.seqlens), o, lse, B, 1, 1, P, wide, px.num_pages, 128,
                         c.scale, 0, ws, nbytes)
    torch.cuda.synchronize()
    O_ref, L_ref = paged_ref(px)
    o64, l64 = bf16_dev_to_f64(o), lse.cpu().numpy()
    empty = x.seqlens == 0
    assert np.all(o64[empty] == 0) and np.all(np.isneginf(l64[empty]))
    keep = np.flatnonzero(~empty)
    assert_bf16(o64[keep], O_ref[keep])
    assert_lse(l64[keep], L_ref[keep])


@pytest.mark.parametrize("P", [16, 64])
@pytest.mark.parametrize("splits", [1, 16])
def test_paged_partition_many_short_sequences(P, splits):
    """The work partition over sequence ends on the paged cache: 70 sequences
    of 0..96 keys (two groups of 64 in the prefix sums), so work items start
    and end inside pages and cross many sequence ends (1 split), or hold one
    block each (16 splits)."""
    _need_gpu()
    B = 70
    c = W.Decode("paged_short", B, 8, 2, 96, 128, 1 / math.sqrt(128), 1, 96, 56)
    x = W.decode_inputs(c, seqlens=[(7 * b) % 97 for b in range(B)])
    px = W.paged_from_decode(x, P, perm_seed=P + splits)
    o, lse = run_paged(px, splits)
    O_ref, L_ref = paged_ref(px)
    o64, l64 = bf16_dev_to_f64(o), lse.cpu().numpy()
    tag = f"P={P} splits={splits}"
    empty = x.seqlens == 0
    assert np.all(o64[empty] == 0) and np.all(np.isneginf(l64[empty])), tag
    keep = np.flatnonzero(~empty)
    assert_bf16(o64[keep], O_ref[keep], tag)
    assert_lse(l64[keep], L_ref[keep], tag)
