"""ctypes loader for libint8lin.so (the C ABI declared in include/int8lin.h).

Loading never falls back to anything: if the shared library is missing the
import of this module raises, naming the build command.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("I8L_LIBRARY", os.path.join(_HERE, "libint8lin.so"))

I8L_F32, I8L_F16, I8L_BF16 = 0, 1, 2
I8L_OK, I8L_EINVAL, I8L_EDTYPE, I8L_ESHAPE, I8L_EWORKSPACE, I8L_EHIP, I8L_EOVERFLOW = 0, -1, -2, -3, -4, -5, -6
I8L_ESCRATCH = -7
I8L_NOALLOC_SCRATCH_BYTES = 64 << 20
I8L_MAX_K = 133144
I8L_MAX_COLS = 262144

# every symbol the header declares, with (restype, argtypes)
_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_int = ctypes.c_int


class ForwardLayout(ctypes.Structure):
    _fields_ = [("count", _sz), ("idx", _sz), ("scale", _sz), ("codes", _sz), ("sub", _sz), ("wsub", _sz),
                ("total", _sz)]


SIGNATURES = {
    "int8_linear_strerror": (ctypes.c_char_p, [_int]),
    "int8_quantize_rowwise_workspace_bytes": (_sz, [_i64, _i64]),
    "int8_quantize_rowwise": (_int, [_vp, _int, _i64, _i64, _f32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]),
    "int8_linear_forward_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "int8_linear_forward_workspace_layout": (_int, [_i64, _i64, _i64, _i32, ctypes.POINTER(ForwardLayout)]),
    "int8_linear_forward": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _i64, _vp, _f32, _i32, _vp, _vp, _vp, _sz,
                                   _vp]),
    "int8_linear_forward_check": (_int, [_vp, _i64, _i64, _i64, _i32, _vp, ctypes.POINTER(_i32)]),
    "int8_linear_forward_plan": (_int, [_int, _i64, _i64, _i64]),
    "int8_linear_forward_noalloc_bytes": (_sz, [_i64, _i64, _i64]),
    "int8_linear_forward_noalloc_max_bytes": (_sz, []),
    "int8_linear_forward_noalloc": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _i64, _vp, _f32, _vp, _vp]),
    "int8_linear_backward_plan": (_int, [_int, _i64, _i64, _i64]),
    "int8_linear_backward_workspace_bytes": (_sz, [_i64, _i64, _int]),
    "int8_linear_backward_input": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "int8_linear_backward_int8_workspace_bytes": (_sz, [_i64, _i64, _int]),
    "int8_linear_backward_input_int8": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _sz,
                                               _vp]),
    "int8_linear_backward_weight": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _vp, _vp]),
    "int8_outlier_flags_words": (_sz, [_i64, _i64]),
    "int8_silu_outlier_flags": (_int, [_vp, _int, _i64, _i64, _f32, _vp, _vp, _sz, _vp]),
    "int8_linear_forward_flagged": (_int, [_vp, _int, _i64, _i64, _vp, _sz, _vp, _vp, _i64, _vp, _i32, _vp, _vp,
                                           _vp, _sz, _vp]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"HIP library not found at {LIB_PATH}; build it with "
            "`python int8_quantized_linear_rowwise_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class Int8LinError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {lib.int8_linear_strerror(code).decode()} (code {code})")


def check(code: int, where: str) -> None:
    if code != I8L_OK:
        raise Int8LinError(code, where)
