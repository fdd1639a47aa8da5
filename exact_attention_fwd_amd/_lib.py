"""ctypes loader for libfa.so (the gfx950 HIP library built in-tree).

torch is imported before the library is opened so that the one HIP runtime
already mapped by torch (soname libamdhip64.so.7) is the one the library
binds to.  A missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_FILE = os.path.join(PKG_DIR, "libfa.so")

FA_F32 = 0
FA_BF16 = 1

STATUS_NAMES = {
    0: "FA_OK",
    1: "FA_ERR_NULL_PTR",
    2: "FA_ERR_BAD_SHAPE",
    3: "FA_ERR_UNSUPPORTED",
    4: "FA_ERR_WORKSPACE",
    5: "FA_ERR_HIP",
    6: "FA_ERR_SCRATCH_TOO_SMALL",
}

_lib = None


def library_path() -> str:
    return _LIB_FILE


def status_name(code: int) -> str:
    return STATUS_NAMES.get(int(code), f"status {code}")


class FaError(RuntimeError):
    def __init__(self, code: int):
        self.code = int(code)
        L = lib()
        msg = L.fa_status_str(self.code).decode()
        if self.code == 5:
            msg += f" ({L.fa_last_hip_error().decode()})"
        super().__init__(msg)


def _declare(L):
    c_int, c_float, c_size, vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    L.fa_status_str.argtypes = [c_int]
    L.fa_status_str.restype = ctypes.c_char_p
    L.fa_last_hip_error.argtypes = []
    L.fa_last_hip_error.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = c_int
    L.fa_forward.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, c_int, c_float, vp]
    L.fa_forward.restype = c_int
    L.fa_backward_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    L.fa_backward_workspace_bytes.restype = c_size
    L.fa_backward.argtypes = [c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, c_size,
                              c_int, c_float, vp]
    L.fa_backward.restype = c_int
    i32p = vp
    L.fa_forward_gqa.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, c_int, c_float, vp]
    L.fa_forward_gqa.restype = c_int
    L.fa_forward_varlen.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, i32p, vp, vp, vp, vp, vp, c_int,
                                    c_float, vp]
    L.fa_forward_varlen.restype = c_int
    L.fa_backward_gqa.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  c_size, c_int, c_float, vp]
    L.fa_backward_gqa.restype = c_int
    L.fa_backward_varlen_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.fa_backward_varlen_workspace_bytes.restype = c_size
    L.fa_backward_varlen.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, i32p, vp, vp, vp, vp, vp, vp,
                                     vp, vp, vp, vp, c_size, c_int, c_float, vp]
    L.fa_backward_varlen.restype = c_int
    L.fa_decode_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    L.fa_decode_workspace_bytes.restype = c_size
    L.fa_decode_paged.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp, c_float, vp,
                                  c_size, vp]
    L.fa_decode_paged.restype = c_int
    L.fa_decode_paged_gqa.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp,
                                      c_float, vp, c_size, vp]
    L.fa_decode_paged_gqa.restype = c_int
    L.fa_decode_static_scratch_bytes.argtypes = []
    L.fa_decode_static_scratch_bytes.restype = c_size
    L.fa_decode_paged_gqa_static.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                             vp, c_float, vp]
    L.fa_decode_paged_gqa_static.restype = c_int
    L.fa_prefill_paged.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp, c_int, c_int, vp, c_int,
                                   vp, vp, vp, c_int, c_float, vp, vp, c_int, c_int, vp]
    L.fa_prefill_paged.restype = c_int
    L.fa_forward_rope.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, vp, c_int,
                                  c_float, vp, vp, c_int, c_int, vp]
    L.fa_forward_rope.restype = c_int


def lib():
    """The loaded library (opened once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_FILE):
            raise RuntimeError(
                f"{_LIB_FILE} is missing: build it with `python -m exact_attention_fwd_amd.build` "
                "(there is no fallback implementation)")
        import torch  # noqa: F401  (maps the HIP runtime first)
        L = ctypes.CDLL(_LIB_FILE)
        _declare(L)
        _lib = L
    return _lib
