"""ctypes loader for libcalibatt.so (built in-tree by build.py).

There is no fallback: if the library is missing or fails to load, every
entry point raises, naming the file and the build command.
"""

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcalibatt.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "calibatt.h")

STATUS = {
    0: "CALIBATT_OK",
    1: "CALIBATT_ERR_NULL",
    2: "CALIBATT_ERR_SHAPE",
    3: "CALIBATT_ERR_DTYPE",
    4: "CALIBATT_ERR_ALIGN",
    5: "CALIBATT_ERR_CSR",
    6: "CALIBATT_ERR_CAPACITY",
    7: "CALIBATT_ERR_UNSUPPORTED",
    8: "CALIBATT_ERR_HIP",
}
BF16, F32 = 0, 1
V_BHLD, V_BHDL = 0, 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

SIGNATURES = {
    "calibatt_sparse_attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _f32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _vp, _vp, _i64, _i32, _vp]),
    "calibatt_sparse_attn_fwd_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _f32, _i32, _i32, _i32,
                                                _i32, _i32, _i32, _vp, _i64, _i32, _vp]),
    "calibatt_dense_attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _i32, _f32, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _vp, _i32, _vp]),
    "calibatt_transpose_v": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "calibatt_block_mass": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp,
                                   _vp]),
    "calibatt_block_mass_single_pass": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                               _vp, _vp, _sz, _vp]),
    "calibatt_block_mass_ws_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "calibatt_compile_masks": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _vp,
                                      ctypes.POINTER(_i64), _vp, _sz, _vp]),
    "calibatt_compile_masks_energy": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _i32, _vp, _vp,
                                             _i64, _vp, ctypes.POINTER(_i64), _vp, _sz, _vp]),
    "calibatt_compile_ws_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "calibatt_share_timesteps": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_double, _vp, _vp,
                                        _vp, _vp, _vp, _i64, ctypes.POINTER(_i32), ctypes.POINTER(_i64), _vp, _sz,
                                        _vp]),
    "calibatt_share_ws_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "calibatt_encode_skip_lists": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i64, _vp, _vp, _i32,
                                          ctypes.POINTER(_i32), ctypes.POINTER(_i32), _vp, _sz, _vp]),
    "calibatt_decode_skip_lists": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i64,
                                          ctypes.POINTER(_i64), _vp, _sz, _vp]),
    "calibatt_skip_ws_bytes": (_sz, [_i32, _i32, _i32]),
    "calibatt_spatial_similarity": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _i32,
                                           _vp, _vp, _vp, _sz, _vp]),
    "calibatt_similarity_ws_bytes": (_sz, [_i32, _i32, _i32]),
    "calibatt_select_repetitive_heads": (_i32, [_vp, _i32, _i32, ctypes.c_double, _vp, ctypes.POINTER(_i32), _vp]),
    "calibatt_anchor_attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _vp, _i32, _vp, _sz, _vp]),
    "calibatt_anchor_ws_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "calibatt_anchor_parts": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "calibatt_build_schedule": (_i32, [_vp, _i32, _i32, _vp, _vp]),
    "calibatt_validate_csr": (_i32, [_vp, _vp, _i32, _i32, _i64]),
    "calibatt_status_string": (ctypes.c_char_p, [_i32]),
    "calibatt_last_error": (ctypes.c_char_p, []),
    "calibatt_version": (_i32, []),
}

_lib = None


class CalibattError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


def load():
    """Load the library once; raise with the build command if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m block_sparse_attention_calibatt_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status):
    if status != 0:
        lib = load()
        msg = lib.calibatt_last_error().decode()
        raise CalibattError(status, msg)


def header_symbols(path=HEADER):
    """Names of the functions include/calibatt.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(calibatt_[a-z0-9_]+)\s*\(", text)))
