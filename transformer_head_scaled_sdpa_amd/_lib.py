"""ctypes declarations of libmha.so (the C ABI in include/mha.h).

No fallback: if the library is missing or fails to load, every call raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmha.so")

MHA_F32 = 0
MHA_BF16 = 1

MHA_OK = 0
MHA_EINVAL = 1
MHA_ENOTSUP = 2
MHA_EWORKSPACE = 3
MHA_EHIP = 4

# Every function the header declares; tests check that each is exported.
EXPORTED = ("sdpa_forward", "sdpa_forward_lse", "sdpa_forward_ex", "sdpa_backward_workspace_bytes", "sdpa_backward",
            "sdpa_backward_lse",
            "sdpa_decode_workspace_bytes", "sdpa_decode", "sdpa_decode_noalloc", "mha_workspace_bytes",
            "mha_workspace_bytes_ex", "mha_forward", "mha_forward_ex", "mha_sublayer_workspace_bytes",
            "mha_sublayer_forward", "mha_backward_workspace_bytes", "mha_backward", "mha_saved_bytes",
            "mha_forward_train", "mha_backward_saved_workspace_bytes", "mha_backward_saved", "mha_status_string",
            "mha_timing_enable",
            "mha_timing_read")


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_longlong), ("h", ctypes.c_longlong), ("l", ctypes.c_longlong)]


class MhaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None


def load():
    """Load libmha.so once; raise ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m transformer_head_scaled_sdpa_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.sdpa_forward.restype = i
    lib.sdpa_forward.argtypes = [i, i, vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                 i, i, i, i, i, i, vp, i, vp]
    lib.sdpa_forward_lse.restype = i
    lib.sdpa_forward_lse.argtypes = [i, i, vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                     i, i, i, i, i, i, vp, i, vp, vp]
    lib.sdpa_forward_ex.restype = i
    lib.sdpa_forward_ex.argtypes = [i, i, vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                    i, i, i, i, i, i, vp, i, i, vp, Strides, vp]
    lib.sdpa_backward_workspace_bytes.restype = sz
    lib.sdpa_backward_workspace_bytes.argtypes = [i, i, i]
    lib.sdpa_backward.restype = i
    lib.sdpa_backward.argtypes = [i, i] + [vp, Strides] * 8 + [i] * 6 + [vp, i, i, vp, sz, vp]
    lib.sdpa_backward_lse.restype = i
    lib.sdpa_backward_lse.argtypes = [i, i] + [vp, Strides] * 8 + [i] * 6 + [vp, i, i, vp, vp, sz, vp]
    lib.sdpa_decode_workspace_bytes.restype = sz
    lib.sdpa_decode_workspace_bytes.argtypes = [i, i, i]
    lib.sdpa_decode.restype = i
    lib.sdpa_decode.argtypes = [i, i, vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                i, i, i, i, i, vp, vp, sz, vp]
    lib.sdpa_decode_noalloc.restype = i
    lib.sdpa_decode_noalloc.argtypes = [i, i, vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                        i, i, i, i, i, vp, vp]
    lib.mha_workspace_bytes.restype = sz
    lib.mha_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.mha_forward.restype = i
    lib.mha_forward.argtypes = [i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                i, i, i, i, i, i, vp, i, vp, sz, vp]
    lib.mha_saved_bytes.restype = sz
    lib.mha_saved_bytes.argtypes = [i, i, i, i, i, i]
    lib.mha_forward_train.restype = i
    lib.mha_forward_train.argtypes = [i, i] + [vp] * 11 + [i] * 6 + [vp, i, vp, sz, vp]
    lib.mha_backward_saved_workspace_bytes.restype = sz
    lib.mha_backward_saved_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.mha_backward_saved.restype = i
    lib.mha_backward_saved.argtypes = [i] + [vp] * 6 + [vp, sz] + [vp] * 11 + [i] * 6 + [vp, i, vp, sz, vp]
    lib.mha_backward_workspace_bytes.restype = sz
    lib.mha_backward_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.mha_backward.restype = i
    lib.mha_backward.argtypes = [i] + [vp] * 20 + [i] * 6 + [vp, i, vp, sz, vp]
    lib.mha_workspace_bytes_ex.restype = sz
    lib.mha_workspace_bytes_ex.argtypes = [i, i, i, i, i, i]
    lib.mha_forward_ex.restype = i
    lib.mha_forward_ex.argtypes = [i, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   i, i, i, i, i, i, vp, i, i, vp, Strides, vp, sz, vp]
    lib.mha_sublayer_workspace_bytes.restype = sz
    lib.mha_sublayer_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.mha_sublayer_forward.restype = i
    lib.mha_sublayer_forward.argtypes = [i, i, vp, vp, vp, vp, i, ctypes.c_float] + [vp] * 9 + [i] * 6 + [
        vp, i, vp, sz, vp]
    lib.mha_status_string.restype = ctypes.c_char_p
    lib.mha_status_string.argtypes = [i]
    lib.mha_timing_enable.restype = i
    lib.mha_timing_enable.argtypes = [i]
    lib.mha_timing_read.restype = i
    lib.mha_timing_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int), i]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mha_status_string(int(status)).decode()
