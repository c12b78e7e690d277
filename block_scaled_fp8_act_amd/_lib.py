"""ctypes declarations of libdsfp8.so (the C ABI in include/dsfp8.h)."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsfp8.so")

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in header order.
SIGNATURES = {
    "dsfp8_abi_version": (_i, []),
    "dsfp8_status_string": (ctypes.c_char_p, [_i]),
    "dsfp8_act_quant": (_i, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _i64, _i, _p]),
    "dsfp8_silu_mul_act_quant": (_i, [_p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p, _i64, _i64, _p, _i64, _i,
                                      _p]),
    "dsfp8_weight_quant": (_i, [_p, _i, _i64, _i64, _i64, _p, _i64, _p, _i64, _i, _p]),
    "dsfp8_weight_dequant": (_i, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p]),
    "dsfp8_gemm": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _i, _p, _sz, _p]),
    "dsfp8_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "dsfp8_grouped_gemm": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p,
                                _i64, _i, _p, _sz, _p]),
    "dsfp8_grouped_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "dsfp8_grouped_gemm_noalloc": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64,
                                        _p, _i64, _i, _p]),
    "dsfp8_gemm_silu_mul_act_quant": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64,
                                           _p, _i64, _i64, _p, _i64, _i, _p]),
    "dsfp8_grouped_gemm_silu_mul_act_quant": (_i, [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _i64,
                                                   _i64, _i64, _p, _i64, _p, _i64, _i64, _p, _i64, _i, _p, _sz,
                                                   _p]),
    "dsfp8_grouped_gemm_silu_mul_act_quant_gather": (_i, [_p, _i64, _i64, _p, _i64, _i64, _p, _p, _i64, _p, _i64,
                                                          _p, _i64, _i64, _i64, _i64, _p, _i64, _p, _i64, _i64, _p,
                                                          _i64, _i, _p, _sz, _p]),
    "dsfp8_act_quant_rows": (_i, [_p, _i64, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64, _i, _p]),
    "dsfp8_moe_route": (_i, [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _sz, _p]),
    "dsfp8_moe_route_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "dsfp8_moe_combine": (_i, [_p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p]),
}

_lib = None


def load():
    """Load libdsfp8.so once; raise if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m block_scaled_fp8_act_amd.build` "
            "(there is no CPU or PyTorch fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
