"""fp64 CPU oracle for exact attention (TEST INFRASTRUCTURE ONLY).

This package is the reference the HIP path is checked against.  It is plain,
slow and written to be read against the pages.  Two implementations of the
same definitions live here:

* ``cpp`` (the oracle): plain C++17 in fp64 (``cpp_oracle.cpp``, built into
  ``liboracle.so`` by ``oracle/build.py`` with g++ and OpenMP), reached through
  ctypes.  It materialises S and P one panel of rows at a time, takes the
  softmax in two passes, and runs every product as a plain loop.  The names
  exported at the package level are these.
* ``numpy_ref``: the same definitions in numpy fp64 (library matrix
  products), kept as a second, independent implementation that the C++ one is
  checked against, plus the one-pass online softmax (``attention_online``)
  whose equality with the two-pass form the pins check, and the FLOP
  convention.

Functions and the passages they follow:

* ``attention_forward`` / ``attention_probs`` -- softmax(scale Q K^T) V with
  LSE = m + ln l.  Standard-attention formula on the FlashAttention (TH)
  page, section on standard attention, and the ledger page's "FLOPs"
  section.
* ``attention_online`` -- the one-pass tiled form with a running max and sum
  (CANN ops-transformer FlashAttention page, the four steps under
  "FlashAttention 的解法"; FlashAttention (TH) page, online softmax).  Never
  the reference for the GPU.
* ``attention_backward`` -- dQ, dK, dV by the chain rule of the forward
  definition (the ledger page names the backward pass by its memory cost).
* ``decode`` / ``decode_paged`` -- one new query against all cached keys
  (ledger page, bandwidth section), over a contiguous or a paged cache (the
  PagedAttention scheme named on the CANN ops-transformer FlashAttention page).
* ``hstu_dense`` / ``hstu_jagged`` -- x = QK^T, x *= alpha, x = silu(x),
  x *= mask / n, O = x V (HSTU page, the Python listing), over packed
  variable-length sequences (optimisation three, jagged tensors).

Who may use it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The library and its Python binding never
import it, and it imports nothing from them.  Every function is pinned by tests
in ``tests/test_oracle_*.py`` against closed forms, invariants, brute force and
library routines, for both implementations.
"""

from . import cpp, numpy_ref  # noqa: F401
from .cpp import (  # noqa: F401
    attention_backward,
    attention_forward,
    attention_probs,
    decode,
    decode_paged,
    hstu_dense,
    hstu_jagged,
)
from .numpy_ref import (  # noqa: F401
    allowed_keys,
    attention_bwd_flops,
    attention_flops,
    attention_online,
    hstu_flops,
    silu,
)
