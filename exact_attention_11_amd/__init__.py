"""Python binding of libfattn: exact attention kernels for MI355X (gfx950).

The functions here only marshal arguments into the C ABI declared in
``include/fattn.h``; every step of the computation runs in the library's HIP
kernels.  Tensor arguments may be torch tensors on the GPU (their
``data_ptr()`` is passed) or raw integer device addresses.  ``stream`` defaults
to torch's current stream on the current device.

A missing or unloadable library raises ``FattnLibraryError``; there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "FattnError",
    "FattnLibraryError",
    "attn_fwd",
    "attn_fwd_f32",
    "attn_fwd_fp8",
    "attn_decode",
    "attn_decode_workspace_bytes",
    "attn_decode_noalloc",
    "attn_decode_paged",
    "attn_hstu_jagged",
    "attn_bwd",
    "attn_bwd_workspace_bytes",
    "fattn_status_string",
    "fattn_last_error",
    "library",
    "library_path",
    "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfattn.so")

EXPORTED_SYMBOLS = (
    "attn_fwd",
    "attn_fwd_f32",
    "attn_fwd_fp8",
    "attn_decode_workspace_bytes",
    "attn_decode",
    "attn_decode_noalloc",
    "attn_decode_paged",
    "attn_hstu_jagged",
    "attn_bwd_workspace_bytes",
    "attn_bwd",
    "fattn_status_string",
    "fattn_last_error",
)

FATTN_OK = 0
FATTN_ERR_INVALID_ARG = 1
FATTN_ERR_UNSUPPORTED = 2
FATTN_ERR_HIP = 3
FATTN_ERR_INTERNAL = 4


class FattnLibraryError(RuntimeError):
    """libfattn.so is missing or cannot be loaded."""


class FattnError(RuntimeError):
    """A libfattn call returned a non-zero status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with {_status_name(status)} ({status}): {message}")
        self.status = status
        self.message = message


_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_SIGNATURES = {
    "attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_fwd_f32": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_fwd_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "attn_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "attn_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "attn_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz,
                               _vp]),
    "attn_hstu_jagged": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _f, _i, _vp]),
    "attn_bwd_workspace_bytes": (_sz, [_i, _i, _i]),
    "attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "fattn_status_string": (ctypes.c_char_p, [_i]),
    "fattn_last_error": (ctypes.c_char_p, []),
}


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """Load libfattn.so (once) and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise FattnLibraryError(
                f"{_LIB_PATH} is not built; run `python -m exact_attention_11_amd.build`")
        try:
            lib = ctypes.CDLL(_LIB_PATH)
        except OSError as e:
            raise FattnLibraryError(f"cannot load {_LIB_PATH}: {e}") from e
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _status_name(status: int) -> str:
    try:
        return library().fattn_status_string(status).decode()
    except FattnLibraryError:
        return str(status)


def fattn_status_string(status: int) -> str:
    return library().fattn_status_string(int(status)).decode()


def fattn_last_error() -> str:
    return library().fattn_last_error().decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != FATTN_OK:
        raise FattnError(fn, status, fattn_last_error())


def attn_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, stream=None):
    """bf16 fused attention; see ``attn_fwd`` in include/fattn.h."""
    st = library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Hkv), int(N),
                            int(d), float(scale), int(causal), _stream(stream))
    _check("attn_fwd", st)


def attn_fwd_f32(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, stream=None):
    """f32 fused attention; see ``attn_fwd_f32`` in include/fattn.h."""
    st = library().attn_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Hkv), int(N),
                                int(d), float(scale), int(causal), _stream(stream))
    _check("attn_fwd_f32", st)


def attn_fwd_fp8(q, k, v, o, lse, descale_q, descale_k, descale_v, B, H, Hkv, N, d, scale, causal, stream=None):
    """FP8 (E4M3) fused attention; see ``attn_fwd_fp8`` in include/fattn.h."""
    st = library().attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(descale_q), _ptr(descale_k),
                                _ptr(descale_v), int(B), int(H), int(Hkv), int(N), int(d), float(scale), int(causal),
                                _stream(stream))
    _check("attn_fwd_fp8", st)


def attn_decode_workspace_bytes(B, H, d, num_splits) -> int:
    return int(library().attn_decode_workspace_bytes(int(B), int(H), int(d), int(num_splits)))


def attn_decode(q, k_cache, v_cache, seqlens_k, o, lse, B, H, Hkv, Lmax, d, scale, num_splits, workspace,
                workspace_bytes, stream=None):
    """Split-KV decode plus LSE combine; see ``attn_decode`` in include/fattn.h."""
    st = library().attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), _ptr(o), _ptr(lse),
                               int(B), int(H), int(Hkv), int(Lmax), int(d), float(scale), int(num_splits),
                               _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("attn_decode", st)


def attn_decode_noalloc(q, k_cache, v_cache, seqlens_k, o, lse, B, H, Hkv, Lmax, d, scale, num_splits, stream=None):
    """attn_decode with the library's static scratch array as its workspace;
    see ``attn_decode_noalloc`` in include/fattn.h."""
    st = library().attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), _ptr(o), _ptr(lse),
                                       int(B), int(H), int(Hkv), int(Lmax), int(d), float(scale), int(num_splits),
                                       _stream(stream))
    _check("attn_decode_noalloc", st)


def attn_decode_paged(q, k_pages, v_pages, block_table, seqlens_k, o, lse, B, H, Hkv, page_size, max_pages_per_seq,
                      num_pages, d, scale, num_splits, workspace, workspace_bytes, stream=None):
    """Split-KV decode over a paged cache; see ``attn_decode_paged`` in include/fattn.h."""
    st = library().attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seqlens_k),
                                     _ptr(o), _ptr(lse), int(B), int(H), int(Hkv), int(page_size),
                                     int(max_pages_per_seq), int(num_pages), int(d), float(scale), int(num_splits),
                                     _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check("attn_decode_paged", st)


def attn_hstu_jagged(q, k, v, o, offsets, B, H, d, max_seqlen, alpha, inv_n, causal, stream=None):
    """Jagged HSTU SiLU attention; see ``attn_hstu_jagged`` in include/fattn.h."""
    st = library().attn_hstu_jagged(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(offsets), int(B), int(H), int(d),
                                    int(max_seqlen), float(alpha), float(inv_n), int(causal), _stream(stream))
    _check("attn_hstu_jagged", st)


def attn_bwd_workspace_bytes(B, H, N) -> int:
    return int(library().attn_bwd_workspace_bytes(int(B), int(H), int(N)))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, N, d, scale, causal, workspace, workspace_bytes,
             stream=None):
    """Gradients of ``attn_fwd`` wrt q, k, v; see ``attn_bwd`` in include/fattn.h."""
    st = library().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                            int(B), int(H), int(Hkv), int(N), int(d), float(scale), int(causal), _ptr(workspace),
                            int(workspace_bytes), _stream(stream))
    _check("attn_bwd", st)
