"""ctypes declarations for libmoe_mi355x.so (mirrors include/moe.h)."""
from __future__ import annotations

import ctypes
import os
import re

from .build import LIB_PATH, INCLUDE

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_SCRATCH_TOO_SMALL = 0, 1, 2, 3, 4
MOE_PERMUTE_NOALLOC_SCRATCH_BYTES = 4 << 20
MOE_DT_F32, MOE_DT_BF16, MOE_DT_F16 = 0, 1, 2
MOE_W_DENSE, MOE_W_INT4_SYM_GROUP, MOE_W_DENSE_NK, MOE_W_DENSE_NK_F16, MOE_W_FP8_E4M3 = 0, 1, 2, 3, 4
MOE_OP_GATE_UP_SWIGLU, MOE_OP_DOWN = 0, 1


class MoeGemmArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("op", "act_dtype", "wfmt", "group_size", "K", "N", "n_groups", "rows_cap", "a_rows",
                 "row_div", "m_hint", "out_dtype")] + \
               [(n, ctypes.c_void_p) for n in
                ("a", "row_index", "group_offsets", "w0", "w1", "s0", "s1", "out")]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


_lib = None


def header_functions() -> list[str]:
    """Names of the functions declared in include/moe.h."""
    with open(os.path.join(INCLUDE, "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def load(path: str = LIB_PATH):
    """Load the HIP library.  Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no CPU or PyTorch fallback")
    L = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    L.moe_abi_version.argtypes, L.moe_abi_version.restype = [], i32
    L.moe_status_string.argtypes, L.moe_status_string.restype = [i32], ctypes.c_char_p
    L.moe_route.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    L.moe_pack_routing.argtypes = [vp, vp, i32, i32, vp, vp]
    L.moe_prepare_router_weights.argtypes = [vp, i32, i32, vp, vp]
    L.moe_router_logits.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, vp]
    L.moe_route_hidden.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    L.moe_route_packed.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
    L.moe_permute_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_permute_workspace_bytes.restype = ctypes.c_size_t
    L.moe_permute.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.moe_permute_noalloc.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp]
    L.moe_grouped_gemm.argtypes = [ctypes.POINTER(MoeGemmArgs), vp]
    L.moe_combine.argtypes = [vp, i32, i32, vp, vp, vp, i32, i32, i32, vp, i32, vp]
    L.moe_prepare_dense_weights.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    L.moe_prepare_dense_weights_f16.argtypes = [vp, i32, i32, i32, vp, vp]
    for fn in ("moe_route", "moe_pack_routing", "moe_route_packed", "moe_permute", "moe_permute_noalloc",
               "moe_prepare_router_weights", "moe_router_logits", "moe_route_hidden",
               "moe_grouped_gemm",
               "moe_combine", "moe_prepare_dense_weights", "moe_prepare_dense_weights_f16"):
        getattr(L, fn).restype = i32
    _lib = L
    return L


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        msg = load().moe_status_string(status).decode()
        raise MoeError(fn, status, msg)
