"""Helpers shared by the tests: device transfer of bf16 bit arrays and the
parity checker (tolerances written here, in one place)."""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from synthgen import bf16_bits_to_f64

# Tolerances on bf16 outputs: max |dO| and mean |dO| (absolute) on every
# compared element; relative Frobenius error and a normalised max error keep
# the check meaningful where outputs are small (decode, HSTU).
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_REL_FRO = 1e-2
BF16_REL_MAX = 2e-2
F32_MAX_ABS = 1e-5
F32_REL_FRO = 1e-6
LSE_MAX_ABS = 1e-3
# Gradients (backward pass): their scale grows with N and the scores, so the
# bound is relative -- Frobenius error and max error, both normalised by the
# reference.  bf16 rounding of P, dS and the outputs gives about 2^-9 per term.
GRAD_REL_FRO = 1e-2
GRAD_REL_MAX = 2e-2
# FP8 prefill: P is rounded to E4M3 before the P V product; each weight's
# relative rounding error is at most 2^-4 (RMS 2^-4/sqrt(3) = 3.6 %), so O's
# relative error stays within a few percent.  The bounds are relative (O's
# scale follows the descales) with ~2x margin over the measured worst case
# (rel_fro 2.6e-2, rel_max 3.5e-2).  LSE uses the unrounded weights and keeps
# the bf16 bound.
FP8_REL_FRO = 5e-2
FP8_REL_MAX = 8e-2


def to_dev_bf16(bits: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(arr: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def bf16_dev_to_f64(t) -> np.ndarray:
    import torch

    return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


@dataclass
class Diff:
    max_abs: float
    mean_abs: float
    rel_fro: float
    rel_max: float
    finite: bool

    def __str__(self):
        return (f"max|d|={self.max_abs:.3e} mean|d|={self.mean_abs:.3e} rel_fro={self.rel_fro:.3e} "
                f"rel_max={self.rel_max:.3e} finite={self.finite}")


def diff(got: np.ndarray, ref: np.ndarray) -> Diff:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    finite = bool(np.all(np.isfinite(got)))
    d = np.abs(got - ref)
    if d.size == 0:
        return Diff(0.0, 0.0, 0.0, 0.0, finite)
    nref = np.linalg.norm(ref)
    mref = np.max(np.abs(ref))
    return Diff(float(d.max()), float(d.mean()),
                float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got)),
                float(d.max() / mref) if mref > 0 else float(d.max()),
                finite)


def bf16_ok(got, ref) -> tuple[bool, Diff]:
    r = diff(got, ref)
    ok = (r.finite and r.max_abs <= BF16_MAX_ABS and r.mean_abs <= BF16_MEAN_ABS
          and r.rel_fro <= BF16_REL_FRO and r.rel_max <= BF16_REL_MAX)
    return ok, r


def f32_ok(got, ref) -> tuple[bool, Diff]:
    r = diff(got, ref)
    return (r.finite and r.max_abs <= F32_MAX_ABS and r.rel_fro <= F32_REL_FRO), r


def lse_ok(got, ref) -> tuple[bool, Diff]:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    same_inf = np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    r = diff(got[fin], ref[fin]) if fin.any() else Diff(0, 0, 0, 0, True)
    return (same_inf and r.finite and r.max_abs <= LSE_MAX_ABS), r


def assert_bf16(got, ref, what=""):
    ok, r = bf16_ok(got, ref)
    assert ok, f"{what}: {r}"
    return r


def assert_grad(got, ref, what=""):
    r = diff(got, ref)
    assert r.finite and r.rel_fro <= GRAD_REL_FRO and r.rel_max <= GRAD_REL_MAX, f"{what}: {r}"
    return r


def assert_fp8(got, ref, what=""):
    r = diff(got, ref)
    assert r.finite and r.rel_fro <= FP8_REL_FRO and r.rel_max <= FP8_REL_MAX, f"{what}: {r}"
    return r


def assert_lse(got, ref, what=""):
    ok, r = lse_ok(got, ref)
    assert ok, f"{what} LSE: {r}"
    return r


def sample_rows(N: int, bm: int = 128, bn: int = 32, stride: int = 61) -> np.ndarray:
    """Rows compared at full size when the oracle cannot do all of them: the
    first and last two query tiles, rows either side of each key-tile
    boundary (where the causal diagonal tile changes; 32-key tiles, which
    include the 64-key tiles' boundaries), and every stride-th row."""
    rows = set(range(0, min(N, 2 * bm)))
    rows |= set(range(max(0, N - 2 * bm), N))
    for t in range(bn, N, bn):
        rows |= {t - 1, t}
    rows |= set(range(0, N, stride))
    return np.array(sorted(r for r in rows if 0 <= r < N), dtype=np.int64)
