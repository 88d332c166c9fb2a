"""ctypes view of libvsa.so (the C ABI declared in include/vsa.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvsa.so")

VSA_F32, VSA_BF16 = 0, 1

STATUS_NAMES = {
    0: "VSA_OK", 1: "VSA_ERR_NULL", 2: "VSA_ERR_SHAPE", 3: "VSA_ERR_HEAD_DIM", 4: "VSA_ERR_DTYPE",
    5: "VSA_ERR_TOPK", 6: "VSA_ERR_ALIGN", 7: "VSA_ERR_WORKSPACE", 8: "VSA_ERR_INDEX",
    9: "VSA_ERR_UNSUPPORTED", 10: "VSA_ERR_HIP", 11: "VSA_ERR_SCALE",
}


class VsaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("heads", ctypes.c_int32), ("T", ctypes.c_int32),
                ("H", ctypes.c_int32), ("W", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("topk", ctypes.c_int32),
                ("list_stride", ctypes.c_int32), ("pool_mode", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("cube_t", ctypes.c_int32), ("cube_h", ctypes.c_int32), ("cube_w", ctypes.c_int32),
                ("kcube_t", ctypes.c_int32), ("kcube_h", ctypes.c_int32), ("kcube_w", ctypes.c_int32)]


_P = ctypes.POINTER(VsaProblem)
_v = ctypes.c_void_p
_sz = ctypes.c_size_t
_i32 = ctypes.c_int32

# name -> (restype, argtypes); every symbol include/vsa.h and include/vsa_probe.h declare.
SIGNATURES = {
    "vsa_tile": (_i32, [_P, _v, _v, _v]),
    "vsa_untile": (_i32, [_P, _v, _v, _v]),
    "vsa_compatible_latent": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _v, _v, _v]),
    "vsa_crop": (_i32, [_P, _v, _i32, _i32, _i32, _v, _v]),
    "vsa_pad": (_i32, [_P, _v, _i32, _i32, _i32, _v, _v]),
    "vsa_status_string": (ctypes.c_char_p, [_i32]),
    "vsa_version": (_i32, []),
    "vsa_max_cubes": (_i32, []),
    "vsa_workspace_bytes": (_sz, [_P, _i32]),
    "vsa_saved_bytes": (_sz, [_P]),
    "vsa_forward": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _sz, _v]),
    "vsa_backward": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _sz, _v]),
    "vsa_pool": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v]),
    "vsa_coarse": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _sz, _v]),
    "vsa_fine_forward": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _sz, _v]),
    "vsa_fine_combine": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _sz, _v]),
    "vsa_fine_combine_noalloc": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v]),
    "vsa_combine": (_i32, [_P, _v, _v, _v, _v, _v, _v]),
    "vsa_combine_backward": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v]),
    "vsa_index_transpose": (_i32, [_P, _v, _v, _v, _v, _v, _sz, _v]),
    "vsa_fine_backward": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v,
                                 _v, _sz, _v]),
    "vsa_coarse_backward": (_i32, [_P, _v, _v, _v, _v, _v, _v, _v, _v, _v, _v, _sz, _v]),
    "vsa_check_lists_host": (_i32, [_P, _v, _v]),
    "vsa_validate_lists": (_i32, [_P, _v, _v, _v, _v]),
    # include/vsa_probe.h: measurement aids
    "vsa_probe_mfma_valu": (_i32, [_i32, _i32, _i32, _i32, _v, _v]),
    "vsa_probe_stream_read": (_i32, [_v, _sz, _i32, _i32, _i32, _v, _v]),
    "vsa_probe_l2_to_lds": (_i32, [_i32, _v, _sz, _i32, _i32, _v, _v]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m block_sparse_video_cube_amd.build` "
                "(the VSA operator has no non-HIP implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class VsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))
        msg = lib().vsa_status_string(status).decode()
        super().__init__(f"{where}: {self.name} ({msg})")


def check(status: int, where: str) -> None:
    if status != 0:
        raise VsaError(status, where)
