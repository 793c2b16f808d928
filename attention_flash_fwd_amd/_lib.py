"""ctypes view of libattn.so (include/attn.h).

The library is loaded after torch so that both share torch's HIP runtime
(libamdhip64.so.7 is resolved by soname to the copy torch already mapped).
There is no fallback: if the library is missing or does not load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK = 0
STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_ALIGN", 3: "ATTN_ERR_SHAPE",
    4: "ATTN_ERR_DTYPE", 5: "ATTN_ERR_UNSUPPORTED", 6: "ATTN_ERR_WORKSPACE", 7: "ATTN_ERR_LAUNCH",
}
ATTN_BF16 = 0
ATTN_F32 = 1
MAX_SPLITS = 256
STATIC_SCRATCH_BYTES = 32 << 20     # ATTN_STATIC_SCRATCH_BYTES

# Every symbol include/attn.h declares.
EXPORTED = ("attn_prefill", "attn_prefill_paged", "attn_decode_paged", "attn_decode_paged_multi",
            "attn_decode_paged_fp8", "attn_decode_paged_noalloc",
            "attn_decode_workspace_bytes", "attn_decode_multi_workspace_bytes",
            "attn_decode_num_splits", "attn_status_string", "attn_abi_version")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


def _declare(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    F = ctypes.c_float
    Z = ctypes.c_size_t
    lib.attn_prefill.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.attn_prefill.restype = I
    lib.attn_prefill_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, P]
    lib.attn_prefill_paged.restype = I
    lib.attn_decode_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P, Z, P]
    lib.attn_decode_paged.restype = I
    lib.attn_decode_paged_noalloc.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P]
    lib.attn_decode_paged_noalloc.restype = I
    lib.attn_decode_paged_multi.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, P, Z, P]
    lib.attn_decode_paged_multi.restype = I
    lib.attn_decode_paged_fp8.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, F, F, P, Z, P]
    lib.attn_decode_paged_fp8.restype = I
    lib.attn_decode_multi_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.attn_decode_multi_workspace_bytes.restype = Z
    lib.attn_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.attn_decode_workspace_bytes.restype = Z
    lib.attn_decode_num_splits.argtypes = [I, I, I, I, I]
    lib.attn_decode_num_splits.restype = I
    lib.attn_status_string.argtypes = [I]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = I
    return lib


def load():
    """Load libattn.so (after torch's HIP runtime); raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- maps torch's libamdhip64 first
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m attention_flash_fwd_amd.build")
    _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(status: int) -> str:
    if _lib is None:
        return STATUS_NAMES.get(status, "unknown")
    return _lib.attn_status_string(int(status)).decode()
