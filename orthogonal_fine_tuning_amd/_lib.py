"""ctypes view of liboft.so (the C ABI in include/oft.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("OFT_LIBRARY") or os.path.join(_HERE, "liboft.so")

OFT_OK, OFT_EINVAL, OFT_ESHAPE, OFT_EDTYPE, OFT_EUNSUPPORTED, OFT_EWORKSPACE, OFT_EHIP = (
    0, -1, -2, -3, -4, -5, -6)
OFT_DT_BF16, OFT_DT_F32 = 0, 1
OFT_W_INT4, OFT_W_FP8_E4M3, OFT_W_BF16, OFT_W_FP4_E2M1, OFT_W_INT4_TILED = 0, 1, 2, 3, 4
OFT_PASS_FWD, OFT_PASS_BWD = 0, 1
OFT_MAX_SEGMENTS = 8
OFT_NOALLOC_SCRATCH_BYTES = 128 << 20


class oft_linear_desc(C.Structure):
    _fields_ = [("M", C.c_int32), ("K", C.c_int32), ("N", C.c_int32), ("x_dtype", C.c_int32),
                ("w_fmt", C.c_int32), ("g", C.c_int32), ("b", C.c_int32), ("n_seg", C.c_int32),
                ("seg", C.c_int32 * OFT_MAX_SEGMENTS)]


class oft_moe_desc(C.Structure):
    _fields_ = [("T", C.c_int32), ("E", C.c_int32), ("k", C.c_int32), ("H", C.c_int32),
                ("I", C.c_int32), ("g", C.c_int32), ("b", C.c_int32), ("chunk", C.c_int32),
                ("renorm", C.c_int32), ("w_fmt", C.c_int32)]


class oft_moe_routing(C.Structure):
    _fields_ = [("topk_idx", C.c_void_p), ("topk_w", C.c_void_p), ("counts", C.c_void_p),
                ("offsets", C.c_void_p), ("perm", C.c_void_p), ("inv_perm", C.c_void_p),
                ("active", C.c_void_p), ("n_active", C.c_void_p),
                ("chunk_of_expert", C.c_void_p)]


_P = C.c_void_p
_I = C.c_int32
_SZ = C.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "oft_abi_version": (_I, []),
    "oft_prof_enable": (_I, [_I]),
    "oft_prof_count": (_I, []),
    "oft_prof_read": (_I, [_I, C.c_char_p, _I, C.POINTER(C.c_float)]),
    "oft_status_str": (C.c_char_p, [_I]),
    "oft_last_hip_error": (_I, []),
    "cayley_build": (_I, [_P, _I, _I, _P, _P, _P]),
    "oft_dequant": (_I, [_I, _I, _I, _I, _P, _P, _P, _P]),
    "oft_pack_int4_tiled": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "oft_linear_workspace_bytes": (_I, [C.POINTER(oft_linear_desc), _I, C.POINTER(_SZ)]),
    "oft_linear_fwd": (_I, [C.POINTER(oft_linear_desc), _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "oft_linear_fwd_base": (_I, [C.POINTER(oft_linear_desc), _P, _P, _P, _P, _P, _SZ, _P]),
    "oft_slots_switch": (_I, [_P, C.c_int32, C.c_int32, _P]),
    "oft_linear_fwd_slots": (_I, [C.POINTER(oft_linear_desc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "oft_moe_router_bwd": (_I, [C.POINTER(oft_moe_desc), _P, _P, _P, _P, _P]),
    "oft_linear_bwd": (_I, [C.POINTER(oft_linear_desc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                            _P]),
    "oft_linear_bwd_noalloc": (_I, [C.POINTER(oft_linear_desc), _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "oft_logprob_diff": (_I, [_I, _I, _P, _P, _P, _P, _P]),
    "oft_moe_workspace_bytes": (_I, [C.POINTER(oft_moe_desc), _I, C.POINTER(_SZ)]),
    "oft_moe_route": (_I, [C.POINTER(oft_moe_desc), _P, C.POINTER(oft_moe_routing), _P, _SZ, _P]),
    "oft_moe_grouped_fwd": (_I, [C.POINTER(oft_moe_desc), _P, _P, _P, _P, _P, _P, _P,
                                 C.POINTER(oft_moe_routing), _P, _P, _P, _SZ, _P]),
    "oft_moe_grouped_fwd_base": (_I, [C.POINTER(oft_moe_desc), _P, _P, _P, _P, _P, _P,
                                      C.POINTER(oft_moe_routing), _P, _P, _P, _SZ, _P]),
    "oft_moe_grouped_bwd": (_I, [C.POINTER(oft_moe_desc), _P, C.POINTER(oft_moe_routing), _P, _P,
                                 _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
}

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load liboft.so once and attach the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it first (python -m orthogonal_fine_tuning_amd.build)")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class OftError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.oft_status_str(status).decode()
        if status == OFT_EHIP:
            msg += f" (hipError {lib.oft_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != OFT_OK:
        raise OftError(status, where)
