"""ctypes loader for libw4a16.so.  Fails loudly when the library is missing:
there is no fallback implementation."""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# W4A16_LIB names another build of the same sources (the host-sanitizer
# check uses it); there is no other implementation to fall back on.
LIB_PATH = os.environ.get("W4A16_LIB") or os.path.join(PKG, "libw4a16.so")

Q4_OK, Q4_ERR_NULL, Q4_ERR_SHAPE, Q4_ERR_GROUP, Q4_ERR_ALIGN, Q4_ERR_HIP, Q4_ERR_CAPACITY = range(7)
ABI_VERSION = 4

# Every symbol the public header declares, with its ctypes signature.
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
SIGNATURES = {
    "q4_abi_version": (ctypes.c_int, []),
    "q4_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "q4_last_hip_error": (ctypes.c_int, []),
    "q4_quantize_pack": (ctypes.c_int, [_p, _i64, _i64, _i32, _i32, _p, _p, _p, _p]),
    "q4_dequant": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i32, _p, _p]),
    "q4_gemv": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, _p]),
    "q4_gemm": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, _p]),
    "q8_quantize_pack": (ctypes.c_int, [_p, _i64, _i64, _i32, _i32, _p, _p, _p, _p]),
    "q8_dequant": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i32, _p, _p]),
    "q8_gemv": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, _p]),
    "q8_gemm": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, _p]),
    "q4_linear_config": (ctypes.c_int, [_i32, _i32, _i64, _i64, _i64, _i32, _p, _p, ctypes.c_char_p, _i64]),
    "kv_quant_tokens": (ctypes.c_int, [_p, _i64, _i32, _i32, _p, _p, _p]),
    "kv_quant_channels": (ctypes.c_int, [_p, _i64, _i32, _i32, _i32, _p, _p, _p]),
    "kv_dequant_tokens": (ctypes.c_int, [_p, _p, _i64, _i32, _p, _p]),
    "kv_dequant_channels": (ctypes.c_int, [_p, _p, _i64, _i32, _i32, _p, _p]),
    "kv_flush_blocks": (ctypes.c_int, [_p, _p, _i64, _i32, _i32, _i32, _p, _i64, _p, _p, _p, _p, _p]),
    "sq_absmax_update_f16": (ctypes.c_int, [_p, _i64, _i32, _p, _p]),
    "sq_absmax_update_f32": (ctypes.c_int, [_p, _i64, _i32, _p, _p]),
    "sq_smooth_factors": (ctypes.c_int, [_p, _p, _i32, ctypes.c_float, _p, _p]),
    "w8a8_quantize_weight": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _p]),
    "w8a8_quantize_act": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _p]),
    "w8a8_gemm": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _p]),
    "gptq_factor_workspace_size": (_i64, [_i64]),
    "gptq_hinv_factor": (ctypes.c_int, [_p, _i64, _i64, ctypes.c_double, _p, _i64, _p, _p]),
    "gptq_quantize_workspace_size": (_i64, [_i64, _i64]),
    "gptq_quantize": (ctypes.c_int, [_p, _p, _i64, _i64, _i32, _i32, _i32, _p, _i64, _p, _p, _p, _p]),
    "gptq_quantize_noalloc": (ctypes.c_int, [_p, _p, _i64, _i64, _i32, _i32, _i32, _p, _p, _p, _p]),
    "gptq_quantize_noalloc_max_bytes": (_i64, []),
    "awq_workspace_size": (_i64, [_i64, _i64, _i64, _i32, _i32]),
    "awq_quantize": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _p, _i64, _p, _p, _p, _p,
                                    _p, _p, _p]),
}


class W4A16Error(RuntimeError):
    """A non-zero status from the library, or the library is unavailable."""

    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise W4A16Error(f"{LIB_PATH} is not built; run `python -m w4a16_dequant_gemv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.q4_abi_version() != ABI_VERSION:
            raise W4A16Error(f"libw4a16 ABI {L.q4_abi_version()} != expected {ABI_VERSION}")
        _LIB = L
    return _LIB


def check(status, what):
    if status != Q4_OK:
        L = lib()
        msg = L.q4_strerror(status).decode()
        if status == Q4_ERR_HIP:
            msg += f" (hipError {L.q4_last_hip_error()})"
        raise W4A16Error(f"{what}: {msg}", status)
