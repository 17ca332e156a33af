"""Loader for libattn.so and its C signatures (ctypes).

The library is the only compute path: if it is missing, importing the binding
fails loudly -- there is no fallback.  torch is imported first so that the
library binds to the HIP runtime torch has already loaded (both carry the
soname libamdhip64.so.7), and device pointers and streams from torch are valid
in it.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch  # noqa: F401  (load torch's HIP runtime before the library)

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
INCLUDE_DIR = os.path.join(os.path.dirname(PKG_DIR), "include")
HEADER_PATH = os.path.join(INCLUDE_DIR, "attn.h")

STATUS_NAMES = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL_PTR",
    2: "ATTN_ERR_BAD_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_MISALIGNED",
    5: "ATTN_ERR_LAUNCH",
    6: "ATTN_ERR_TOO_LARGE",
    7: "ATTN_ERR_SCRATCH",
}
ATTN_F16, ATTN_BF16 = 0, 1

_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

SIGNATURES = {
    "attn_status_string": (ctypes.c_char_p, [_c_int]),
    "attn_prefill_fwd": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                  _c_int, _vp]),
    "attn_prefill_varlen_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _vp, _vp]),
    "attn_decode_num_splits": (_c_int, [_c_int, _c_int, _c_int]),
    "attn_decode_q4_num_splits": (_c_int, [_c_int, _c_int, _c_int]),
    "attn_decode_chunk_len": (_c_int, [_c_int, _c_int]),
    "attn_decode_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "attn_decode_splitk": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                    _c_int, _vp, _vp, _vp, _vp]),
    "attn_decode_splitk_paged": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                          _vp]),
    "attn_decode_splitk_q4": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_float, _c_int, _c_int, _vp, _vp, _vp, _vp]),
    "attn_decode_splitk_q4_paged": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _c_int,
                                             _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _vp, _vp,
                                             _vp, _vp]),
    "attn_kv_quantize_q4": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _vp, _vp]),
    "attn_decode_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                     _c_int, _vp, _vp]),
    "attn_merge_partials": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _c_int, _vp]),
    # measurement helpers (include/attn_calibrate.h)
    "attn_calib_mfma_bf16": (_c_int, [_vp, _c_int, _c_int, _vp]),
    "attn_calib_read": (_c_int, [_vp, _c_size, _vp, _c_int, _vp]),
}


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{fn} returned {self.status_name}")


def header_functions(paths=None):
    """Names of the functions the headers under ``include/`` declare."""
    if paths is None:
        paths = sorted(os.path.join(INCLUDE_DIR, f) for f in os.listdir(INCLUDE_DIR) if f.endswith(".h"))
    names = []
    for path in paths:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names += re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)
    return names


_LIB = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m exact_attention_flashattention_amd.build` "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        raise AttnError(fn, status)
