"""ctypes loader for libtwl.so (the C ABI in include/twl.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libtwl.so")

TWL_OK = 0
STATUS_NAMES = {0: "TWL_OK", 1: "TWL_EINVAL", 2: "TWL_ESHAPE", 3: "TWL_EALIGN",
                4: "TWL_EDEVICE", 5: "TWL_EHIP"}
PATH_AUTO, PATH_GEMM, PATH_GEMV, PATH_GEMV_DOT4, PATH_GEMV_MFMA = 0, 1, 2, 3, 4
OUT_F32, OUT_ACC_I32, OUT_BF16 = 0, 1, 2
HBLOCK, GROUP, MAX_K, GEMV_MAX_M = 1024, 128, 65536, 24
NOALLOC_SCRATCH_BYTES = 32 << 20

# (name, restype, argtypes) for every symbol include/twl.h declares
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIZE = ctypes.c_size_t
_INT = ctypes.c_int
SIGNATURES = [
    ("twl_rotate_quant_act", _INT, [_P, _P, _I64, _I64, _P, _P, _P]),
    ("twl_silu_mul_rotate_quant_act", _INT, [_P, _P, _I64, _I64, _P, _P, _P]),
    ("twl_rotate_act_bf16", _INT, [_P, _P, _I64, _I64, _P, _P]),
    ("twl_reference_linear_bf16", _INT, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    ("twl_pack_ternary", _INT, [_P, _P, _I64, _I64, _P, _P, _P, _P, _P]),
    ("twl_packed_bytes", _SIZE, [_I64, _I64]),
    ("twl_workspace_bytes", _SIZE, [_I64, _I64, _I64]),
    ("twl_ternary_linear", _INT, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _SIZE, _P]),
    ("twl_ternary_linear_acc", _INT, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _SIZE, _P]),
    ("twl_ternary_linear_ex", _INT,
     [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _INT, _INT, _P, _SIZE, _P]),
    ("twl_ternary_linear_noalloc", _INT,
     [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _INT, _INT, _P]),
    ("twl_plan_info", _INT, [_I64, _I64, _I64, _INT, _P]),
    ("twl_rotate_quant_linear", _INT,
     [_P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _P, _P, _P, _INT, _P, _SIZE, _P]),
    ("twl_rotate_quant_linear_fused", _INT, [_I64, _I64, _I64]),
    ("twl_last_error", ctypes.c_char_p, []),
    ("twl_abi_version", _INT, []),
]

_lib = None


class TwlError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {message}")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the library with typed prototypes."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it first with "
            "`python -m ternary_weight_linear_block_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != TWL_OK:
        msg = load().twl_last_error()
        raise TwlError(status, where, msg.decode() if msg else "")
