"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws random numbers and rounds them to the storage type; it holds
none of the attention arithmetic.  Both the fp64 oracle and the HIP path take
their inputs from here so that they see the very same bits.

Recipe (one stream per tensor):

* generator: numpy's PCG64.  A tensor is drawn in chunks of 2^22 values;
  chunk c of tensor ``tensor_id`` uses ``SeedSequence([seed, tensor_id, c])``
  (tensor ids: Q=1, K=2, V=3, lengths=4), so every tensor and chunk has its
  own stream, drawing one never shifts another, and chunks can be drawn in
  parallel threads;
* values: ``sigma * standard_normal`` drawn in float32 (numpy's float32
  ziggurat), then rounded to bfloat16 (round-to-nearest-even) where the
  workload stores bf16;
* lengths: integers uniform on the closed interval ``[lo, hi]``.

The value distributions and shapes follow the workloads the pages describe:
``[batch, heads, seq_len, head_dim]`` with i.i.d. normal entries (the usage
example on the Ascend FlashAttention page, "在昇腾NPU上怎么用"), and packed
jagged sequences with per-sequence lengths (the HSTU page, optimisation three
"Jagged变长张量").
"""

from __future__ import annotations

import os

import numpy as np

TENSOR_Q = 1
TENSOR_K = 2
TENSOR_V = 3
TENSOR_LENGTHS = 4
TENSOR_DO = 5  # upstream gradient dO of the backward pass
TENSOR_PAGES = 6  # physical page order of a paged KV cache


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    NaN inputs map to the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns as float64."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


E4M3_MAX = 448.0  # largest finite OCP FP8 E4M3 value


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP FP8 E4M3 (1 sign, 4 exponent bits with bias
    7, 3 mantissa bits, no infinities; nearest, ties to even); return uint8 bits.

    Magnitudes beyond 448 saturate to +-448; NaN maps to 0x7F.
    """
    x = np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(np.nan_to_num(x, nan=0.0)), E4M3_MAX)
    # exponent of the binade (normal numbers from 2^-6); subnormals share 2^-6's spacing 2^-9
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = np.exp2(e - 3)                  # spacing of representable values in the binade
    q = np.rint(a / step) * step           # round half to even on the exact quotient
    # rounding up may reach the next binade: recompute its fields from q
    with np.errstate(divide="ignore"):
        e2 = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = q >= 2.0 ** -6
    e2 = np.where(normal, np.clip(e2, -6, 8), -6)
    mant = np.where(normal, q / np.exp2(e2) - 1.0, q / 2.0 ** -6) * 8.0
    exp_field = np.where(normal, e2 + 7, 0)
    bits = (exp_field.astype(np.uint8) << np.uint8(3)) | np.rint(mant).astype(np.uint8)
    bits = bits | sign
    bits[np.isnan(np.asarray(x))] = np.uint8(0x7F)
    return bits


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 bit patterns as float64 (0x7F / 0xFF are NaN)."""
    b = np.ascontiguousarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = s * v
    return np.where((b & 0x7F) == 0x7F, np.nan, v)


def normal_e4m3(seed: int, tensor_id: int, shape, scale_axes: int = 2, sigma: float = 1.0):
    """i.i.d. N(0, sigma^2) values (as drawn by normal_f32) quantised to E4M3
    with one float32 descale per leading ``scale_axes``-index (e.g. per
    (batch, head)): descale = amax / 448, bits = round(x / descale).  The
    tensor's value is bits * descale.  Returns (uint8 bits, float32 descale)."""
    x = normal_f32(seed, tensor_id, shape, sigma)
    lead = shape[:scale_axes]
    flat = x.reshape(int(np.prod(lead)), -1)
    amax = np.abs(flat).max(axis=1)
    descale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    bits = f32_to_e4m3_bits((flat / descale[:, None]).astype(np.float32))
    return bits.reshape(shape), descale.reshape(lead)


_CHUNK = 1 << 22


def _chunk_rng(seed: int, tensor_id: int, c: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id), int(c)])))


def _draw(seed: int, tensor_id: int, shape, sigma: float, to_bf16: bool) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if to_bf16 else np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        s0, s1 = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        z = _chunk_rng(seed, tensor_id, c).standard_normal(s1 - s0, dtype=np.float32)
        if sigma != 1.0:
            z *= np.float32(sigma)
        out[s0:s1] = f32_to_bf16_bits(z) if to_bf16 else z

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        from concurrent.futures import ThreadPoolExecutor

        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1, nchunks)) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def normal_f32(seed: int, tensor_id: int, shape, sigma: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, sigma^2) values in float32."""
    return _draw(seed, tensor_id, shape, sigma, False)


def normal_bf16(seed: int, tensor_id: int, shape, sigma: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, sigma^2) values rounded to bfloat16; returns uint16 bit patterns."""
    return _draw(seed, tensor_id, shape, sigma, True)


def uniform_lengths(seed: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` integers uniform on the closed interval [lo, hi] (int32)."""
    g = _rng(seed, TENSOR_LENGTHS)
    return g.integers(lo, hi, size=count, endpoint=True).astype(np.int32)


def offsets_from_lengths(lengths) -> np.ndarray:
    """Exclusive prefix sum of lengths: int32 array of size len(lengths)+1."""
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    if off[-1] > np.iinfo(np.int32).max:
        raise ValueError("total length does not fit int32 offsets")
    return off.astype(np.int32)


BF16_QNAN = np.uint16(0x7FC0)
