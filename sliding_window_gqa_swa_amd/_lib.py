"""ctypes loader for libswa.so (the C ABI declared in include/swa.h).

There is no fallback: if the library is missing or fails to load, every
entry point raises.  Build it with ``python -m sliding_window_gqa_swa_amd.build``.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libswa.so")

SWA_OK = 0
SWA_EINVAL = -1
SWA_EUNSUPPORTED = -2
SWA_ELAUNCH = -3
SWA_EWORKSPACE = -4
SWA_ESCRATCH = -5

SWA_BF16 = 0
SWA_F32 = 1
SWA_CAUSAL = 0
SWA_BLOCKWISE = 1
SWA_META_ERR = -2 ** 31

# (name, restype, argtypes) of every exported symbol
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t
SIGNATURES = {
    "swa_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "swa_prefill_chunk": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _I,
                                         _I, _F, _P]),
    "swa_prefill_backward_workspace_bytes": (_S, [_I, _I]),
    "swa_prefill_lse": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _I, _I,
                                       _F, _P]),
    "swa_prefill_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _I,
                                            _I, _I, _I, _I, _I, _F, _P, _S, _P]),
    "swa_decode_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "swa_decode": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _F, _P, _S, _P]),
    "swa_decode_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _F, _P,
                                       _S, _P]),
    "swa_decode_step_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I,
                                               _I, _F, _P]),
    "swa_cache_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "swa_cache_compact": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "swa_cache_roll": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "swa_strerror": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


class SwaError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = lib().swa_strerror(code).decode()
        super().__init__("%s failed: %s (code %d)" % (fn, msg, code))


def lib():
    """The loaded library (loads on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libswa.so is not built (expected at %s); run "
                               "python -m sliding_window_gqa_swa_amd.build" % LIB_PATH)
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(fn_name, rc):
    if rc != SWA_OK:
        raise SwaError(fn_name, rc)
