"""Workload recipes: shapes, seeds and value distributions of each case.

No attention arithmetic lives here -- only what to draw and how to lay it out.

The five workloads (sizes from the pages' examples where they give them):

* ``tiny_f32``      B=1, H=2, N=256, d=64, fp32, non-causal, scale 1/8.
* ``prefill_d64``   B=1, H=32, N=4096, d=64, bf16, causal, scale 1/8 -- the
  ``[1, 32, 4096, 64]`` tensors of the Ascend FlashAttention page's usage
  example ("在昇腾NPU上怎么用").
* ``prefill_d128``  B=8, H=32, N=4096, d=128, bf16, scale 1/sqrt(128), causal
  and non-causal -- the batch 8 / seq 4096 / head_dim 128 setting of the CANN
  ops-transformer page's measurement table.
* ``prefill_long``  B=1, H=32, N=32768, d=128, bf16, causal.
* ``prefill_d256``  B=4, H=32, N=4096, d=256, bf16, scale 1/16, causal (the
  widest head dimension the forward kernel takes).
* ``decode_gqa``    B=16, H=32, Hkv=8, Lmax=32768, lengths uniform on
  [16384, 32768], d=128, bf16, scale 1/sqrt(128).  Cache rows at or beyond a
  sequence's length hold NaN so that reading them would show.
* ``hstu_jagged``   16 sequences, lengths uniform on [512, 4096], H=4, d=64,
  bf16 0.5*N(0,1), alpha=1/8, 1/n=1/4096, causal -- the (16, 4, 4096, 64)
  shape of the HSTU page's measurements, made jagged as in its optimisation
  three.

Seeds: workload k of the list above (tiny=0 ... hstu=4) uses seed 1000+k;
``prefill_long`` shares seed 1002 with ``prefill_d128``; ``prefill_d256``
uses seed 1003 (as the decode workload: a different shape, so different
draws).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import (
    BF16_QNAN,
    TENSOR_K,
    TENSOR_PAGES,
    TENSOR_Q,
    TENSOR_V,
    bf16_bits_to_f64,
    e4m3_bits_to_f64,
    normal_bf16,
    normal_e4m3,
    normal_f32,
    offsets_from_lengths,
    uniform_lengths,
)


@dataclass(frozen=True)
class Dense:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    scale: float
    causal: bool
    dtype: str  # "f32" or "bf16"
    seed: int
    sigma: float = 1.0


@dataclass(frozen=True)
class Decode:
    name: str
    B: int
    H: int
    Hkv: int
    Lmax: int
    d: int
    scale: float
    len_lo: int
    len_hi: int
    seed: int
    sigma: float = 1.0


@dataclass(frozen=True)
class Jagged:
    name: str
    nseq: int
    H: int
    d: int
    len_lo: int
    len_hi: int
    alpha: float
    inv_n: float
    causal: bool
    seed: int
    sigma: float = 0.5


TINY_F32 = Dense("tiny_f32", 1, 2, 2, 256, 64, 1.0 / 8.0, False, "f32", 1000)
PREFILL_D64 = Dense("prefill_d64", 1, 32, 32, 4096, 64, 1.0 / 8.0, True, "bf16", 1001)
PREFILL_D128_CAUSAL = Dense("prefill_d128_causal", 8, 32, 32, 4096, 128, 1.0 / math.sqrt(128.0), True, "bf16", 1002)
PREFILL_D128_FULL = Dense("prefill_d128_noncausal", 8, 32, 32, 4096, 128, 1.0 / math.sqrt(128.0), False, "bf16", 1002)
PREFILL_LONG = Dense("prefill_long", 1, 32, 32, 32768, 128, 1.0 / math.sqrt(128.0), True, "bf16", 1002)
PREFILL_D256 = Dense("prefill_d256", 4, 32, 32, 4096, 256, 1.0 / 16.0, True, "bf16", 1003)
PREFILL_FP8 = Dense("prefill_fp8_d128_causal", 8, 32, 32, 4096, 128, 1.0 / math.sqrt(128.0), True, "fp8", 1006)
DECODE_GQA = Decode("decode_gqa", 16, 32, 8, 32768, 128, 1.0 / math.sqrt(128.0), 16384, 32768, 1003)
HSTU_JAGGED = Jagged("hstu_jagged", 16, 4, 64, 512, 4096, 1.0 / 8.0, 1.0 / 4096.0, True, 1004)


@dataclass
class DenseInputs:
    case: Dense
    q: np.ndarray  # bf16 bits (uint16) or float32, [B, H, N, d]
    k: np.ndarray  # [B, Hkv, N, d]
    v: np.ndarray

    def f64(self, name: str, index=()) -> np.ndarray:
        a = getattr(self, name)[index]
        return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def dense_inputs(c: Dense) -> DenseInputs:
    qs = (c.B, c.H, c.N, c.d)
    ks = (c.B, c.Hkv, c.N, c.d)
    draw = normal_bf16 if c.dtype == "bf16" else normal_f32
    return DenseInputs(
        c,
        draw(c.seed, TENSOR_Q, qs, c.sigma),
        draw(c.seed, TENSOR_K, ks, c.sigma),
        draw(c.seed, TENSOR_V, ks, c.sigma),
    )


@dataclass
class DecodeInputs:
    case: Decode
    q: np.ndarray  # bf16 bits [B, H, d]
    k: np.ndarray  # bf16 bits [B, Hkv, Lmax, d]; rows >= seqlens[b] are NaN
    v: np.ndarray
    seqlens: np.ndarray  # int32 [B]


def decode_inputs(c: Decode, seqlens=None) -> DecodeInputs:
    if seqlens is None:
        seqlens = uniform_lengths(c.seed, c.B, c.len_lo, c.len_hi)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    q = normal_bf16(c.seed, TENSOR_Q, (c.B, c.H, c.d), c.sigma)
    k = normal_bf16(c.seed, TENSOR_K, (c.B, c.Hkv, c.Lmax, c.d), c.sigma)
    v = normal_bf16(c.seed, TENSOR_V, (c.B, c.Hkv, c.Lmax, c.d), c.sigma)
    for b in range(c.B):
        k[b, :, seqlens[b]:, :] = BF16_QNAN
        v[b, :, seqlens[b]:, :] = BF16_QNAN
    return DecodeInputs(c, q, k, v, seqlens)


@dataclass
class Fp8DenseInputs:
    case: Dense
    q: np.ndarray         # E4M3 bits (uint8) [B, H, N, d]
    k: np.ndarray         # [B, Hkv, N, d]
    v: np.ndarray
    descale_q: np.ndarray  # float32 [B, H]: value = bits * descale
    descale_k: np.ndarray  # float32 [B, Hkv]
    descale_v: np.ndarray

    def f64(self, name: str, index=()) -> np.ndarray:
        bits = getattr(self, name)[index]
        ds = getattr(self, "descale_" + name)[index[:2] if isinstance(index, tuple) else index]
        return e4m3_bits_to_f64(bits) * ds.astype(np.float64)[..., None, None]


def fp8_dense_inputs(c: Dense) -> Fp8DenseInputs:
    """Q, K, V drawn as normal_f32 (sigma) and quantised to E4M3 with one
    descale per (batch, head)."""
    q, dq = normal_e4m3(c.seed, TENSOR_Q, (c.B, c.H, c.N, c.d), 2, c.sigma)
    k, dk = normal_e4m3(c.seed, TENSOR_K, (c.B, c.Hkv, c.N, c.d), 2, c.sigma)
    v, dv = normal_e4m3(c.seed, TENSOR_V, (c.B, c.Hkv, c.N, c.d), 2, c.sigma)
    return Fp8DenseInputs(c, q, k, v, dq, dk, dv)


@dataclass
class PagedDecodeInputs:
    base: DecodeInputs       # the same cache, contiguous
    page_size: int
    k_pages: np.ndarray      # bf16 bits [num_pages, Hkv, page_size, d]
    v_pages: np.ndarray
    block_table: np.ndarray  # int32 [B, max_pages]
    num_pages: int


def paged_from_decode(x: DecodeInputs, page_size: int, spare_pages: int = 64, perm_seed: int = 0
                      ) -> PagedDecodeInputs:
    """Scatter a contiguous decode cache into pages of ``page_size`` rows, in a
    seeded random physical order.  Spare pages (never referenced) and rows past
    Lmax are NaN, so a wrong page or row read shows up in the output."""
    c = x.case
    P = int(page_size)
    ppseq = (c.Lmax + P - 1) // P
    num_pages = c.B * ppseq + spare_pages
    rng = np.random.default_rng(np.random.SeedSequence([c.seed, TENSOR_PAGES, perm_seed]))
    perm = rng.permutation(num_pages).astype(np.int32)
    table = perm[:c.B * ppseq].reshape(c.B, ppseq)

    def scatter(cache):
        pad = ppseq * P - c.Lmax
        if pad:
            cache = np.concatenate([cache, np.full(cache.shape[:2] + (pad, c.d), BF16_QNAN, np.uint16)], axis=2)
        pages = np.full((num_pages, c.Hkv, P, c.d), BF16_QNAN, dtype=np.uint16)
        pages[table.reshape(-1)] = (cache.reshape(c.B, c.Hkv, ppseq, P, c.d).transpose(0, 2, 1, 3, 4)
                                    .reshape(c.B * ppseq, c.Hkv, P, c.d))
        return pages

    return PagedDecodeInputs(x, P, scatter(x.k), scatter(x.v), table, num_pages)


@dataclass
class JaggedInputs:
    case: Jagged
    q: np.ndarray  # bf16 bits [T, H, d]
    k: np.ndarray
    v: np.ndarray
    lengths: np.ndarray  # int32 [nseq]
    offsets: np.ndarray  # int32 [nseq + 1]
    max_seqlen: int = field(default=0)


def jagged_inputs(c: Jagged, lengths=None) -> JaggedInputs:
    if lengths is None:
        lengths = uniform_lengths(c.seed, c.nseq, c.len_lo, c.len_hi)
    lengths = np.asarray(lengths, dtype=np.int32)
    offsets = offsets_from_lengths(lengths)
    T = int(offsets[-1])
    shape = (T, c.H, c.d)
    return JaggedInputs(
        c,
        normal_bf16(c.seed, TENSOR_Q, shape, c.sigma),
        normal_bf16(c.seed, TENSOR_K, shape, c.sigma),
        normal_bf16(c.seed, TENSOR_V, shape, c.sigma),
        lengths,
        offsets,
        int(lengths.max()) if lengths.size else 0,
    )
