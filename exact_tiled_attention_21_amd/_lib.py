"""ctypes view of libfa.so (include/fa.h). Loading needs no GPU."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F16, FA_BF16 = 0, 1
FA_MAX_SPLITS = 256
STATUS = {0: "FA_OK", 1: "FA_ERR_NULLPTR", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADS", 4: "FA_ERR_HEADDIM",
          5: "FA_ERR_DTYPE", 6: "FA_ERR_SPLITS", 7: "FA_ERR_WORKSPACE", 8: "FA_ERR_LAUNCH",
          9: "FA_ERR_ALIGN", 10: "FA_ERR_SCALE", 11: "FA_ERR_SCRATCH"}
FA_NOALLOC_SCRATCH_BYTES = 32 << 20
EXPORTS = ("fa_fwd", "fa_fwd_window", "fa_fwd_varlen", "fa_decode_workspace_bytes", "fa_decode_splitkv",
           "fa_decode_splitkv_noalloc", "fa_decode_splitkv_paged", "fa_bwd_workspace_bytes", "fa_bwd", "fa_bwd_window", "fa_bwd_varlen",
           "fa_status_str")

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_str(status)})")


def load(path: str = LIB_PATH):
    """Loads the library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with "
                                "`python -m exact_tiled_attention_21_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.fa_fwd.restype = I
    lib.fa_fwd_window.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P]
    lib.fa_fwd_window.restype = I
    lib.fa_fwd_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P]
    lib.fa_fwd_varlen.restype = I
    lib.fa_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_decode_workspace_bytes.restype = S
    lib.fa_decode_splitkv.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P, S, P]
    lib.fa_decode_splitkv.restype = I
    lib.fa_decode_splitkv_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P]
    lib.fa_decode_splitkv_noalloc.restype = I
    lib.fa_decode_splitkv_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F, I, P, S, P]
    lib.fa_decode_splitkv_paged.restype = I
    lib.fa_bwd_workspace_bytes.argtypes = [I, I, I]
    lib.fa_bwd_workspace_bytes.restype = S
    lib.fa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, S, P]
    lib.fa_bwd.restype = I
    lib.fa_bwd_window.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P, S, P]
    lib.fa_bwd_window.restype = I
    lib.fa_bwd_varlen.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P, S, P]
    lib.fa_bwd_varlen.restype = I
    lib.fa_status_str.argtypes = [I]
    lib.fa_status_str.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    try:
        return load().fa_status_str(status).decode()
    except Exception:  # pragma: no cover - message only
        return "?"
