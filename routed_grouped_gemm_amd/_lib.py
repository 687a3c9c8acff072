"""ctypes declarations of libmoe's C ABI (include/moe.h). Loading only: no
function here computes anything; every call goes to the HIP library."""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(6)
MOE_FMT_MXFP4, MOE_FMT_MXFP8 = 0, 1
MOE_ROUTE_RENORM = 1 << 0
MOE_WEIGHT_AT_COMBINE = 1 << 1
MOE_W1_WRITE_TRANSPOSE = 1 << 2
MOE_SCALE_RULE_CEIL = 1 << 3
MOE_GEMM_STREAMED = 1 << 8
MOE_GEMM_TILED = 1 << 9
MOE_GEMM_PASS = 1 << 12
MOE_LAYER_SEPARATE_KERNELS = 1 << 10
MOE_LAYER_TOKEN_RING = 1 << 11
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class moe_weights(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("G", C.c_int32), ("N", C.c_int32), ("K", C.c_int32),
                ("is_w1", C.c_int32), ("reserved", C.c_int32), ("data", C.c_void_p),
                ("bytes", C.c_size_t)]


MOE_ACT_SWIGLU, MOE_ACT_GEGLU, MOE_ACT_SRELU = 0, 1, 2


class moe_epilogue(C.Structure):
    _fields_ = [("act", C.c_int32), ("beta", C.c_float), ("limit", C.c_float), ("reserved", C.c_int32),
                ("bias", C.c_void_p), ("save_pre", C.c_void_p)]


class moe_layer_args(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("T", C.c_int32), ("E_tot", C.c_int32), ("k", C.c_int32),
                ("e0", C.c_int32), ("E_loc", C.c_int32), ("xq", C.c_void_p), ("xs", C.c_void_p),
                ("H", C.c_int32), ("I", C.c_int32), ("w1", C.POINTER(moe_weights)),
                ("w2", C.POINTER(moe_weights)), ("shared_w1", C.POINTER(moe_weights)),
                ("shared_w2", C.POINTER(moe_weights)), ("flags", C.c_uint32),
                ("hTq", C.c_void_p), ("hTs", C.c_void_p), ("out", C.c_void_p),
                ("epi", C.POINTER(moe_epilogue))]


P, I32, U32, SZ = C.c_void_p, C.c_int32, C.c_uint32, C.c_size_t
WP = C.POINTER(moe_weights)
EP = C.POINTER(moe_epilogue)

# name -> (restype, argtypes), in the order of include/moe.h
SIGNATURES = {
    "moe_status_string": (C.c_char_p, [I32]),
    "moe_version": (C.c_char_p, []),
    "moe_prepacked_size": (SZ, [I32, I32, I32, I32]),
    "moe_prepack_weights": (I32, [P, P, I32, I32, I32, I32, I32, P, SZ, P]),
    "moe_quantize_mx": (I32, [P, I32, I32, I32, U32, P, P, P]),
    "moe_hbm_read_probe": (I32, [P, SZ, P, P]),
    "moe_route": (I32, [P, I32, I32, I32, U32, P, P, P]),
    "moe_permute_workspace_size": (SZ, [I32, I32, I32]),
    "moe_permute": (I32, [P, P, I32, I32, I32, I32, I32, P, P, I32, P, P, P, P, P, P, P, P, P, SZ, P]),
    "moe_transposed_ld": (I32, [I32, I32]),
    "moe_grouped_workspace_size": (SZ, [I32, I32, I32, I32]),
    "moe_grouped_w1": (I32, [WP, WP, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, EP, U32, P, P, P,
                             P, P, SZ, P]),
    "moe_backward_workspace_size": (SZ, [I32, I32, I32, I32]),
    "moe_grouped_w1_backward": (I32, [WP, WP, P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, EP, U32,
                                      P, P, P, P, P, P, SZ, P]),
    "moe_grouped_w2": (I32, [WP, WP, P, P, P, P, I32, I32, I32, I32, U32, P, P, SZ, P]),
    "moe_combine": (I32, [P, P, P, I32, I32, I32, P, P]),
    "moe_layer_workspace_size": (SZ, [I32, I32, I32, I32, I32, I32, I32, U32]),
    "moe_layer": (I32, [C.POINTER(moe_layer_args), P, SZ, P]),
    "moe_layer_noalloc": (I32, [C.POINTER(moe_layer_args), P]),
    "moe_layer_workspace_offsets": (I32, [I32, I32, I32, I32, I32, I32, I32, U32, C.POINTER(SZ)]),
}

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libmoe.so and declare every exported signature. Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libmoe.so not found at {path}: run python routed_grouped_gemm_amd/build.py")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib
