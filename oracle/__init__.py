"""fp64 CPU oracle for exact attention (TEST INFRASTRUCTURE ONLY).

This package is the reference the HIP path is checked against.  It is plain,
slow and written to be read against the pages:

* ``attention_forward`` -- softmax(Q K^T * scale) V with the n x n score and
  probability matrices materialised, two passes over each row (max, then
  exponentials and their sum).  Definition: the standard-attention formula on
  the FlashAttention (TH) page, section on the problem of standard attention,
  and the ledger page's "FLOPs" section (S = QK^T/sqrt(d), O = PV).
* ``attention_online`` -- the one-pass tiled form with a running max and a
  running sum of exponentials (CANN ops-transformer FlashAttention page, the
  four steps under "FlashAttention 的解法"; FlashAttention (TH) page, section
  "online softmax").  It exists only so that its equality with the two-pass
  form can be pinned; it is never the reference for the GPU.
* ``attention_backward`` -- the gradients dQ, dK, dV of the forward
  definition for a given dO (chain rule, all n x n matrices materialised);
  the pages name the backward pass only by its memory cost (ledger page,
  memory section).
* ``decode`` -- one new query against all cached keys (ledger page,
  bandwidth section, the decode formula s = q^T k_j, o = sum_j p_j v_j).
* ``decode_paged`` -- ``decode`` over a paged cache: the pages of each
  sequence gathered in logical order through its block table (the
  PagedAttention scheme named on the CANN ops-transformer FlashAttention page).
* ``hstu_jagged`` -- HSTU pointwise attention, x = QK^T, x *= alpha,
  x = silu(x), x *= mask / n, O = x V (HSTU page, the Python listing under
  "先搞懂：HSTU到底难在哪"), over packed variable-length sequences
  (optimisation three, "Jagged变长张量").

Who may use it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The library and its Python binding never
import it, and it imports nothing from them.  Every function here is pinned by
tests in ``tests/test_oracle_*.py`` against closed forms, invariants and
library routines.
"""

from .attention import (  # noqa: F401
    allowed_keys,
    attention_backward,
    attention_bwd_flops,
    attention_flops,
    attention_forward,
    attention_online,
    attention_probs,
    decode,
    decode_paged,
    hstu_dense,
    hstu_flops,
    hstu_jagged,
    silu,
)
