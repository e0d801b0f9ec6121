"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws random numbers and rounds them to the storage type; it holds
none of the attention arithmetic.  Both the fp64 oracle and the HIP path take
their inputs from here so that they see the very same bits.

Recipe (one stream per tensor):

* generator: numpy's PCG64 seeded with ``SeedSequence([seed, tensor_id])``
  (tensor ids: Q=1, K=2, V=3, lengths=4), so each tensor has its own stream
  and drawing one tensor never shifts another;
* values: ``sigma * standard_normal`` drawn in float64, rounded to float32
  (round-to-nearest-even), then to bfloat16 (round-to-nearest-even) where the
  workload stores bf16;
* lengths: integers uniform on the closed interval ``[lo, hi]``.

The value distributions and shapes follow the workloads the pages describe:
``[batch, heads, seq_len, head_dim]`` with i.i.d. normal entries (the usage
example on the Ascend FlashAttention page, "在昇腾NPU上怎么用"), and packed
jagged sequences with per-sequence lengths (the HSTU page, optimisation three
"Jagged变长张量").
"""

from __future__ import annotations

import numpy as np

TENSOR_Q = 1
TENSOR_K = 2
TENSOR_V = 3
TENSOR_LENGTHS = 4


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


def normal_f32(seed: int, tensor_id: int, shape, sigma: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, sigma^2) values rounded to float32."""
    g = _rng(seed, tensor_id)
    n = int(np.prod(shape))
    # Draw in chunks to bound the float64 temporary for large tensors.
    out = np.empty(n, dtype=np.float32)
    chunk = 1 << 24
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = (g.standard_normal(e - s) * sigma).astype(np.float32)
    return out.reshape(shape)


def normal_bf16(seed: int, tensor_id: int, shape, sigma: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, sigma^2) values rounded to bfloat16; returns uint16 bit patterns."""
    return f32_to_bf16_bits(normal_f32(seed, tensor_id, shape, sigma))


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
