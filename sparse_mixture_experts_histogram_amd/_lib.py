"""ctypes view of ``libmoe_mi355x.so`` (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's
gfx950 kernels.  If the library is missing the import of any entry point
raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import c_double, c_int, c_int32, c_int64, c_size_t, c_void_p, c_char_p, POINTER

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MOE_F32, MOE_BF16 = 0, 1
PATH_AUTO, PATH_PREFILL, PATH_DECODE = 0, 1, 2
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP", -5: "MOE_ERR_TOO_LARGE"}
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES


SCORING_SOFTMAX, SCORING_SIGMOID = 0, 1
WEIGHTS_RENORM, WEIGHTS_RAW = 0, 1
EXPERTS_DENSE, EXPERTS_MXFP4, EXPERTS_MXFP8 = 0, 1, 2
ABI_VERSION = 5
FLAG_MX_LINE_ROWS = 1    # MOE_FLAG_MX_LINE_ROWS


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", c_int64), ("d", c_int32), ("E", c_int32), ("k", c_int32),
                ("ffn", c_int32), ("n_shared", c_int32), ("ffn_shared", c_int32),
                ("dtype", c_int32), ("y_dtype", c_int32), ("path", c_int32),
                ("scoring", c_int32), ("weighting", c_int32), ("expert_format", c_int32),
                ("flags", c_int32), ("capacity_factor", c_double)]


class MoeMxScales(ctypes.Structure):
    _fields_ = [("up", c_void_p), ("gate", c_void_p), ("down", c_void_p),
                ("s_up", c_void_p), ("s_gate", c_void_p), ("s_down", c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


_lib = None


def header_symbols():
    """Names of the functions include/moe.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def lib():
    """Load the library once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m sparse_mixture_experts_histogram_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    D = POINTER(MoeDesc)
    L.moe_abi_version.restype = c_int
    L.moe_abi_version.argtypes = []
    if L.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {L.moe_abi_version()}, the binding "
                          f"expects {ABI_VERSION}; rebuild the library")
    L.moe_status_str.restype = c_char_p
    L.moe_status_str.argtypes = [c_int]
    L.moe_validate.restype = c_int
    L.moe_validate.argtypes = [D]
    L.moe_workspace_size.restype = c_int
    L.moe_workspace_size.argtypes = [D, POINTER(c_size_t)]
    L.moe_resolve_path.restype = c_int
    L.moe_resolve_path.argtypes = [D]
    L.moe_grouped_rows.restype = c_int64
    L.moe_grouped_rows.argtypes = [D]
    V = c_void_p
    L.moe_forward.restype = c_int
    L.moe_forward.argtypes = [D, V, V, V, V, V, V, V, V, V, V, V, V, V, V, c_size_t, V]
    L.moe_forward_noalloc.restype = c_int
    L.moe_forward_noalloc.argtypes = [D, V, V, V, V, V, V, V, V, V, V, V, V, V, V]
    L.moe_forward_mx.restype = c_int
    L.moe_forward_mx.argtypes = [D, V, V, V, V, V, V, V, V, V, POINTER(MoeMxScales), V, V, V, V,
                                 V, c_size_t, V, V]
    L.moe_forward_timed.restype = c_int
    L.moe_forward_timed.argtypes = [D, V, V, V, V, V, V, V, V, V, V, V, V, V, V, c_size_t, V, V]
    L.moe_route.restype = c_int
    L.moe_route.argtypes = [D, V, V, V, V, V, V, c_size_t, V]
    L.moe_dispatch.restype = c_int
    L.moe_dispatch.argtypes = [D, V, V, V, V, V, V, c_size_t, V]
    L.moe_experts.restype = c_int
    L.moe_experts.argtypes = [D, V, V, V, V, V, V, V, V, V, V, V, c_size_t, V]
    L.moe_combine.restype = c_int
    L.moe_combine.argtypes = [D, V, V, V, V, V, V]
    _lib = L
    return L
