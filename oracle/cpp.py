"""ctypes front end of the C++ fp64 oracle (TEST INFRASTRUCTURE ONLY).

The arithmetic lives in ``cpp_oracle.cpp``: S and P materialised per row
panel, a two-pass softmax, plain product loops, OpenMP over (batch, head,
panel).  These functions only convert arguments to contiguous float64 /
int64 arrays, call it, and return float64 arrays.  The signatures match those
of ``numpy_ref`` so that the pins run against both implementations.

Each function takes an optional ``counts`` dict; when given, ``counts["macs"]``
receives the multiply-adds the C++ product loops executed.
"""

from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_d = ctypes.c_double
_int = ctypes.c_int

_SIGS = {
    "oracle_attention_forward": [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _d, _int, _p, _i64, _p, _p,
                                 _p, _p],
    "oracle_decode": [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _d, _p, _p, _p],
    "oracle_decode_paged": [_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _d, _p, _p, _p],
    "oracle_hstu_jagged": [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _d, _d, _int, _p, _p],
    "oracle_attention_backward": [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _d, _int, _p, _p, _p, _p],
    "oracle_set_threads": [_int],
    "oracle_max_threads": [],
}


def library() -> ctypes.CDLL:
    """Load liboracle.so, building it with the host compiler if it is absent."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                from .build import build_oracle

                build_oracle(verbose=False)
            lib = ctypes.CDLL(_LIB_PATH)
            for name, args in _SIGS.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = _int if name == "oracle_max_threads" else None
            _lib = lib
    return _lib


def max_threads() -> int:
    return int(library().oracle_max_threads())


def set_threads(n: int) -> None:
    library().oracle_set_threads(int(n))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i64a(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _store(counts, macs):
    if counts is not None:
        counts["macs"] = int(macs.value)


def attention_forward(q, k, v, scale: float, causal: bool, rows=None, *, counts=None):
    """O = softmax(scale * Q K^T) V and LSE = m + ln l (natural log).

    q ``[B, H, Nq, d]``; k ``[B, Hkv, Nk, d]``; v ``[B, Hkv, Nk, dv]``.
    ``rows`` optionally selects query rows (same for every (b, h)); the result
    then has ``len(rows)`` rows.  Causal: row i sees keys j <= i.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    if k.shape != (B, Hkv, Nk, d) or v.shape[:3] != (B, Hkv, Nk):
        raise ValueError("shape mismatch between q, k and v")
    r = None if rows is None else _i64a(rows)
    if r is not None and r.size and (r.min() < 0 or r.max() >= Nq):
        raise ValueError("rows out of range")
    nr = Nq if r is None else r.size
    O = np.zeros((B, H, nr, dv))
    L = np.zeros((B, H, nr))
    macs = ctypes.c_int64(0)
    if B * H * nr > 0:
        library().oracle_attention_forward(_ptr(q), _ptr(k), _ptr(v), B, H, Hkv, Nq, Nk, d, dv, float(scale),
                                           int(bool(causal)), None if r is None else _ptr(r), nr, _ptr(O), _ptr(L),
                                           None, ctypes.byref(macs))
    _store(counts, macs)
    return O, L


def attention_probs(q, k, scale: float, causal: bool, *, counts=None):
    """The materialised probability matrix P of one head: q ``[Nq, d]``, k ``[Nk, d]``."""
    q, k = _f64(q), _f64(k)
    Nq, d = q.shape
    Nk = k.shape[0]
    v = np.zeros((Nk, 1))
    O = np.zeros((1, 1, Nq, 1))
    L = np.zeros((1, 1, Nq))
    P = np.zeros((1, 1, Nq, Nk))
    macs = ctypes.c_int64(0)
    if Nq > 0:
        library().oracle_attention_forward(_ptr(q), _ptr(k), _ptr(v), 1, 1, 1, Nq, Nk, d, 1, float(scale),
                                           int(bool(causal)), None, Nq, _ptr(O), _ptr(L), _ptr(P),
                                           ctypes.byref(macs))
    _store(counts, macs)
    return P[0, 0]


def decode(q, k_cache, v_cache, seqlens, scale: float, *, counts=None):
    """One query per (sequence, head) against cache rows [0, L_b).

    q ``[B, H, d]``; caches ``[B, Hkv, Lmax, d]``; seqlens ``[B]``.
    Returns O ``[B, H, dv]`` and LSE ``[B, H]`` (-inf for an empty history).
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, H, d = q.shape
    Hkv, Lmax, dv = kc.shape[1], kc.shape[2], vc.shape[3]
    sl = _i64a(seqlens)
    O = np.zeros((B, H, dv))
    L = np.zeros((B, H))
    macs = ctypes.c_int64(0)
    if B * H > 0:
        library().oracle_decode(_ptr(q), _ptr(kc), _ptr(vc), _ptr(sl), B, H, Hkv, Lmax, d, dv, float(scale),
                                _ptr(O), _ptr(L), ctypes.byref(macs))
    _store(counts, macs)
    return O, L


def decode_paged(q, k_pages, v_pages, block_table, seqlens, scale: float, *, counts=None):
    """Decode over a paged cache: pages ``[num_pages, Hkv, P, d]``, block_table
    ``[B, max_pages]`` (logical page p of sequence b is physical page
    ``block_table[b, p]``), seqlens ``[B]``."""
    q, kp, vp = _f64(q), _f64(k_pages), _f64(v_pages)
    B, H, d = q.shape
    Hkv, P, dv = kp.shape[1], kp.shape[2], vp.shape[3]
    tab = _i64a(block_table)
    sl = _i64a(seqlens)
    maxp = tab.shape[1]
    if np.any(np.minimum(sl, P * maxp) > 0):
        used = [tab[b, :(int(min(sl[b], P * maxp)) + P - 1) // P] for b in range(B)]
        if any(u.size and (u.min() < 0 or u.max() >= kp.shape[0]) for u in used):
            raise ValueError("block table entry out of range")
    O = np.zeros((B, H, dv))
    L = np.zeros((B, H))
    macs = ctypes.c_int64(0)
    if B * H > 0:
        library().oracle_decode_paged(_ptr(q), _ptr(kp), _ptr(vp), _ptr(tab), _ptr(sl), B, H, Hkv, P, maxp, d, dv,
                                      float(scale), _ptr(O), _ptr(L), ctypes.byref(macs))
    _store(counts, macs)
    return O, L


def hstu_jagged(q, k, v, offsets, alpha: float, inv_n: float, causal: bool, *, counts=None):
    """HSTU pointwise attention over packed sequences.

    q, k ``[T, H, d]``, v ``[T, H, dv]``; sequence b owns rows
    ``[offsets[b], offsets[b+1])``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, d = q.shape
    dv = v.shape[2]
    off = _i64a(offsets)
    if off.size < 1 or off[0] != 0 or np.any(np.diff(off) < 0) or off[-1] > T:
        raise ValueError("offsets must start at 0, be non-decreasing and end within T")
    O = np.zeros((T, H, dv))
    macs = ctypes.c_int64(0)
    if off.size > 1:
        library().oracle_hstu_jagged(_ptr(q), _ptr(k), _ptr(v), _ptr(off), off.size - 1, H, d, dv, float(alpha),
                                     float(inv_n), int(bool(causal)), _ptr(O), ctypes.byref(macs))
    _store(counts, macs)
    return O


def hstu_dense(q, k, v, alpha: float, inv_n: float, causal: bool, *, counts=None):
    """HSTU attention of one dense sequence and head: q, k ``[L, d]``, v ``[L, dv]``."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    L = q.shape[0]
    O = hstu_jagged(q[:, None], k[:, None], v[:, None], [0, L], alpha, inv_n, causal, counts=counts)
    return O[:, 0]


def attention_backward(q, k, v, do, scale: float, causal: bool, *, counts=None):
    """Gradients (dQ, dK, dV) of O = softmax(scale Q K^T) V for a given dO.

    q, do ``[B, H, N, d]``; k, v ``[B, Hkv, N, d]``.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    if v.shape != k.shape or do.shape != q.shape:
        raise ValueError("shape mismatch")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    macs = ctypes.c_int64(0)
    if B * H * N > 0:
        library().oracle_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(do), B, H, Hkv, N, d, float(scale),
                                            int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), ctypes.byref(macs))
    _store(counts, macs)
    return dq, dk, dv
