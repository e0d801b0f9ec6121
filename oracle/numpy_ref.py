"""fp64 reference implementations (TEST INFRASTRUCTURE ONLY; see package doc).

Arrays are float64 numpy arrays holding the exact values of the inputs (the
bf16 or fp32 bits decoded without rounding).  Layouts:

* dense attention: q ``[B, H, N, d]``, k and v ``[B, Hkv, N, d]``;
  query head h reads key/value head ``h // (H // Hkv)`` (grouped-query
  attention, named as a KV-cache reduction on the ledger page, bandwidth
  section; the grouping of consecutive heads is this oracle's reading);
* decode: q ``[B, H, d]``, caches ``[B, Hkv, Lmax, d]``, lengths ``[B]``;
* jagged HSTU: q, k, v ``[T, H, d]`` with ``offsets[B+1]``.

Where the pages leave something open, the reading taken is stated at the
function that depends on it.
"""

from __future__ import annotations

import numpy as np

# Rows handled per materialised panel.  Rows are independent under the
# definition, so computing them in panels changes nothing; it only bounds the
# size of the S and P panels (R x N fp64 each).
_PANEL_ELEMS = 1 << 22


def allowed_keys(i: int, n_keys: int, causal: bool) -> np.ndarray:
    """Key indices query row i may attend to.

    Causal reading: the lower-triangular mask of the HSTU page's in-kernel mask
    section (blocks before the diagonal fully visible, the aligned block
    lower-triangular, later blocks skipped) with the diagonal kept, i.e. j <= i.
    """
    if causal:
        return np.arange(min(i + 1, n_keys))
    return np.arange(n_keys)


def _score_panel(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * q_rows @ k^T (materialised, fp64)."""
    return scale * (q_rows @ k.T)


def _mask_panel(S: np.ndarray, rows: np.ndarray, causal: bool) -> np.ndarray:
    """Set s_ij = -inf where key j is not visible from row i."""
    if causal:
        cols = np.arange(S.shape[1])
        S = np.where(cols[None, :] <= rows[:, None], S, -np.inf)
    return S


def _softmax_two_pass(S: np.ndarray):
    """Row softmax in two passes: the row max, then exponentials and their sum.

    Returns (P, m, l) with P = exp(S - m) / l, m the row max and l the sum of
    exp(S - m).  A fully masked row (all -inf) gets P = 0, m = -inf, l = 0.
    """
    m = S.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    E = np.exp(S - m_safe[:, None])
    l = E.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        P = np.where(l[:, None] > 0, E / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return P, m, l


def attention_probs(q: np.ndarray, k: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """The full probability matrix P = softmax(scale * q k^T) of one head.

    q ``[Nq, d]``, k ``[Nk, d]``; returns ``[Nq, Nk]``.
    """
    rows = np.arange(q.shape[0])
    S = _mask_panel(_score_panel(q, k, scale), rows, causal)
    P, _, _ = _softmax_two_pass(S)
    return P


def attention_forward(q, k, v, scale: float, causal: bool, rows=None):
    """Exact attention O = softmax(scale * Q K^T) V and LSE = m + ln(l).

    q ``[B, H, N, d]``; k, v ``[B, Hkv, N, d]``.  ``rows`` optionally selects
    the query rows to compute (same rows for every (b, h)); the result then
    has shape ``[B, H, len(rows), d]`` and ``[B, H, len(rows)]``.

    LSE reading: the natural-log log-sum-exp of the scaled, unmasked scores of
    the row, i.e. ln of the sum of exponentials that the online method keeps
    beside the running max (FlashAttention (TH) page, "online softmax").
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    group = H // Hkv
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    Nk = k.shape[2]
    O = np.zeros((B, H, rows.size, v.shape[3]), dtype=np.float64)
    L = np.zeros((B, H, rows.size), dtype=np.float64)
    panel = max(1, _PANEL_ELEMS // max(Nk, 1))
    for b in range(B):
        for h in range(H):
            g = h // group
            for p0 in range(0, rows.size, panel):
                pr = rows[p0:p0 + panel]
                S = _mask_panel(_score_panel(q[b, h, pr], k[b, g], scale), pr, causal)
                P, m, l = _softmax_two_pass(S)
                O[b, h, p0:p0 + pr.size] = P @ v[b, g]
                with np.errstate(divide="ignore"):
                    L[b, h, p0:p0 + pr.size] = m + np.log(l)
    return O, L


def attention_backward(q, k, v, do, scale: float, causal: bool):
    """Gradients (dQ, dK, dV) of O = softmax(scale * Q K^T) V for a given dO.

    q and do ``[B, H, N, d]``; k, v ``[B, Hkv, N, d]``.  Returns fp64 arrays
    of the shapes of q, k and v.  The pages name the backward pass only by
    its cost (ledger page, memory section: training keeps n x n backward
    intermediates besides S and P); this is the chain rule of the forward
    definition, written out per head with every n x n matrix materialised:

        P = softmax(scale * Q K^T) (masked as in the forward)
        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij
        dS = P * (dP - D)            (softmax Jacobian, row by row)
        dQ = scale * dS K
        dK = scale * dS^T Q

    Grouped-query attention: a key/value head's gradients are the sums over
    the query heads that read it.  A fully masked row contributes nothing.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    group = H // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            g = h // group
            S = _mask_panel(_score_panel(q[b, h], k[b, g], scale), rows, causal)
            P, _, _ = _softmax_two_pass(S)
            dv[b, g] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, g].T
            D = (P * dP).sum(axis=1)
            dS = P * (dP - D[:, None])
            dq[b, h] = scale * (dS @ k[b, g])
            dk[b, g] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


def attention_online(q, k, v, scale: float, causal: bool, block: int):
    """One-pass tiled attention with a running max and running sum (one head).

    q ``[N, d]``, k and v ``[Nk, d]``.  Keys are visited in blocks of ``block``
    columns.  For each block: update the running row max with the block's
    max; rescale the previously accumulated weights and output by
    exp(m_old - m_new); add the block's exponentials to the running sum and
    its weighted values to the output.  After the last block the output is
    divided by the running sum.  (CANN ops-transformer FlashAttention page,
    steps 1-4 under "FlashAttention 的解法"; FlashAttention (TH) page, "online
    softmax".)
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, Nk = q.shape[0], k.shape[0]
    rows = np.arange(N)
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    acc = np.zeros((N, v.shape[1]))
    for c0 in range(0, Nk, block):
        cols = np.arange(c0, min(Nk, c0 + block))
        S = scale * (q @ k[cols].T)
        if causal:
            S = np.where(cols[None, :] <= rows[:, None], S, -np.inf)
        m_new = np.maximum(m, S.max(axis=1))
        m_ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - m_ref)
        Pt = np.exp(S - m_ref[:, None])
        l = alpha * l + Pt.sum(axis=1)
        acc = alpha[:, None] * acc + Pt @ v[cols]
        m = m_new
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = m + np.log(l)
    return O, lse


def decode(q, k_cache, v_cache, seqlens, scale: float):
    """Decode attention: each query row attends to all cached rows [0, L_b).

    q ``[B, H, d]``; caches ``[B, Hkv, Lmax, d]``; seqlens ``[B]``.
    Returns O ``[B, H, d]`` and LSE ``[B, H]``.

    Reading of the ledger page's decode formula (s_{n+1,j} = q^T k_j over the
    history, o = sum_j p_j v_j): the cache already holds the current token, so
    the query attends to every valid cache row and no causal mask applies.
    Rows at or beyond L_b are never read.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, d = q.shape
    Hkv = k_cache.shape[1]
    group = H // Hkv
    O = np.zeros((B, H, v_cache.shape[3]))
    L = np.zeros((B, H))
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:  # empty history: no visible key, O = 0 and LSE = -inf
            L[b] = -np.inf
            continue
        for h in range(H):
            g = h // group
            kk = np.asarray(k_cache[b, g, :n], dtype=np.float64)
            vv = np.asarray(v_cache[b, g, :n], dtype=np.float64)
            S = scale * (q[b, h][None, :] @ kk.T)
            P, m, l = _softmax_two_pass(S)
            O[b, h] = (P @ vv)[0]
            with np.errstate(divide="ignore"):
                L[b, h] = m[0] + np.log(l[0])
    return O, L


def decode_paged(q, k_pages, v_pages, block_table, seqlens, scale: float):
    """Decode over a paged cache: gather each sequence's pages in logical order,
    then ``decode``.

    q ``[B, H, d]``; pages ``[num_pages, Hkv, P, d]``; block_table
    ``[B, max_pages]`` (logical page p of sequence b is physical page
    ``block_table[b, p]``); seqlens ``[B]``.

    The paged cache is the PagedAttention scheme that the CANN ops-transformer
    FlashAttention page names under KV-cache management (Kwon et al. 2023 in
    the FlashAttention (TH) page's bibliography); paging changes where keys
    live, not what attention computes, so the result is plain decode on the
    gathered rows [0, L_b).  Pages past the last one holding a valid row are
    not read.
    """
    B, H, d = np.asarray(q).shape
    P = k_pages.shape[2]
    O = np.zeros((B, H, v_pages.shape[3]))
    L = np.zeros((B, H))
    for b in range(B):
        n = int(seqlens[b])
        used = block_table[b, :(n + P - 1) // P]
        # [pages, Hkv, P, d] -> [Hkv, pages * P, d], rows in logical order
        if n == 0:  # empty history, as in decode
            L[b] = -np.inf
            continue
        kb = np.concatenate([k_pages[p] for p in used], axis=1)
        vb = np.concatenate([v_pages[p] for p in used], axis=1)
        Ob, Lb = decode(np.asarray(q)[b:b + 1], kb[None, :, :n], vb[None, :, :n], np.array([n]), scale)
        O[b], L[b] = Ob[0], Lb[0]
    return O, L


def silu(x):
    """SiLU(x) = x * sigmoid(x) = x / (1 + e^{-x})."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def hstu_dense(q, k, v, alpha: float, inv_n: float, causal: bool):
    """HSTU pointwise attention of one dense sequence and head.

    q, k, v ``[L, d]``.  In the order of the HSTU page's listing:
    x = q k^T; x *= alpha; x = silu(x); x *= mask / n; O = x v.
    ``inv_n`` is 1/n; ``mask`` is lower-triangular including the diagonal
    when ``causal`` (in-kernel mask section), else all ones.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L = q.shape[0]
    x = q @ k.T
    x = x * alpha
    x = silu(x)
    mask = np.tril(np.ones((L, L))) if causal else np.ones((L, L))
    x = x * (mask * inv_n)
    return x @ v


def hstu_jagged(q, k, v, offsets, alpha: float, inv_n: float, causal: bool):
    """HSTU attention over packed sequences (no padding, no cross-sequence terms).

    q, k, v ``[T, H, d]``; sequence b owns rows [offsets[b], offsets[b+1]).
    Each (sequence, head) is computed exactly as ``hstu_dense``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, d = q.shape
    O = np.zeros((T, H, v.shape[2]))
    offsets = np.asarray(offsets, dtype=np.int64)
    for b in range(offsets.size - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        if e <= s:
            continue
        for h in range(H):
            O[s:e, h] = hstu_dense(q[s:e, h], k[s:e, h], v[s:e, h], alpha, inv_n, causal)
    return O


def attention_flops(B: int, H: int, N: int, d: int, causal: bool) -> int:
    """FLOP count by the ledger page's convention ("FLOPs" section).

    Two products, QK^T and PV, each 2 n^2 d (one multiply and one add per
    multiply-add), 4 n^2 d per head.  Causal skipping of the tiles above the
    diagonal halves it (HSTU page, in-kernel mask: "saves half the compute"),
    so causal is counted as 2 n^2 d per head.
    """
    per_head = 4 * N * N * d
    if causal:
        per_head //= 2
    return B * H * per_head


def attention_bwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> int:
    """Backward FLOPs by the same convention: five products of 2 n^2 d each
    (the score recompute QK^T, dP = dO V^T, dV = P^T dO, dQ = dS K and
    dK = dS^T Q), 10 n^2 d per head, halved when causal."""
    per_head = 10 * N * N * d
    if causal:
        per_head //= 2
    return B * H * per_head


def hstu_flops(lengths, H: int, d: int, causal: bool) -> int:
    """Same convention for jagged HSTU: sum over sequences of 4 L^2 d per head,
    halved when causal."""
    total = 0
    for L in np.asarray(lengths, dtype=np.int64):
        total += 4 * int(L) * int(L) * d
    if causal:
        total //= 2
    return H * total
