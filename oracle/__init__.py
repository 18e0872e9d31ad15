"""CPU oracle for one device's share of a routed sparse MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
The library's product path never does; the oracle shares no code with it.  The arithmetic lives
in plain C (``oracle.c``, built with gcc, no fast-math, no FMA contraction); this module only
marshals numpy arrays through ctypes.  What each function follows is stated in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
DENSE, INT4, FP8 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                        "-shared", "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _LayerArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("T", "H", "I", "k", "e_first", "e_local", "act", "wfmt", "group_size", "shared_I")] + \
               [(n, ctypes.c_void_p) for n in
                ("x", "ids", "w", "wg", "wu", "wd", "sg", "su", "sd", "shg", "shu", "shd")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.orc_exp_ref.argtypes, L.orc_exp_ref.restype = [ctypes.c_float], ctypes.c_float
        L.orc_exp_ref_array.argtypes, L.orc_exp_ref_array.restype = [vp, vp, i64], None
        L.orc_route.argtypes, L.orc_route.restype = [vp, i32, i32, i32, vp, vp], None
        L.orc_router_logits.argtypes, L.orc_router_logits.restype = [vp, i32, vp, vp, i32, i32, i32, vp], None
        L.orc_pack.argtypes, L.orc_pack.restype = [vp, vp, i32, i32, vp], None
        L.orc_unpack.argtypes, L.orc_unpack.restype = [vp, i32, i32, vp, vp], None
        L.orc_permute.argtypes, L.orc_permute.restype = [vp, i32, i32, i32, i32, vp, vp, vp], i32
        L.orc_bf16_to_double.argtypes, L.orc_bf16_to_double.restype = [ctypes.c_uint16], ctypes.c_double
        L.orc_int4_nibble.argtypes, L.orc_int4_nibble.restype = [ctypes.c_int32, i32], i32
        L.orc_fp8_e4m3_to_double.argtypes, L.orc_fp8_e4m3_to_double.restype = [ctypes.c_uint8], ctypes.c_double
        L.orc_expand_matrix.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp]
        L.orc_expand_matrix.restype = None
        L.orc_layer.argtypes, L.orc_layer.restype = [ctypes.POINTER(_LayerArgs), vp, i32, vp], None
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def exp_ref(d) -> np.ndarray:
    d = np.ascontiguousarray(d, dtype=np.float32)
    out = np.empty_like(d)
    lib().orc_exp_ref_array(_p(d), _p(out), d.size)
    return out


def route(logits: np.ndarray, k: int):
    """Top-k routing with renormalised weights -> (ids int32 [T][k], w float32 [T][k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().orc_route(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def router_logits(x: np.ndarray, wr: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """Router projection: fp32 logits [T][E] = fp32(sum_h x[t][h] wr[h][e]) (+ bias[e] in fp32),
    summed in double.  x is bf16 bits (uint16) or fp32 [T][H]; wr fp32 [H][E]."""
    act = 1 if x.dtype == np.uint16 else 0
    x = np.ascontiguousarray(x, dtype=np.uint16 if act else np.float32)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    T, H = x.shape
    E = wr.shape[1]
    assert wr.shape[0] == H
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, E), np.float32)
    lib().orc_router_logits(_p(x), act, _p(wr), _p(b), T, H, E, _p(out))
    return out


def pack(ids: np.ndarray, w: np.ndarray) -> np.ndarray:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, k = ids.shape
    blob = np.empty((2, T, k), np.int32)
    lib().orc_pack(_p(ids), _p(w), T, k, _p(blob))
    return blob


def unpack(blob: np.ndarray):
    blob = np.ascontiguousarray(blob, dtype=np.int32)
    _, T, k = blob.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().orc_unpack(_p(blob), T, k, _p(ids), _p(w))
    return ids, w


def permute(blob: np.ndarray, e_first: int, e_local: int):
    """-> (sorted_pairs[:n_loc], group_offsets [e_local+1], pair_pos [T*k])."""
    blob = np.ascontiguousarray(blob, dtype=np.int32)
    _, T, k = blob.shape
    sp = np.full(T * k, -1, np.int32)
    off = np.empty(e_local + 1, np.int32)
    pp = np.empty(T * k, np.int32)
    n = lib().orc_permute(_p(blob), T, k, e_first, e_local, _p(sp), _p(off), _p(pp))
    return sp[:n].copy(), off, pp


def bf16_to_double(b: int) -> float:
    return lib().orc_bf16_to_double(int(b))


def fp8_e4m3_to_double(code: int) -> float:
    return lib().orc_fp8_e4m3_to_double(int(code) & 0xFF)


def int4_nibble(word: int, i: int) -> int:
    return lib().orc_int4_nibble(ctypes.c_int32(int(np.int32(np.uint32(word & 0xFFFFFFFF)))).value, i)


def expand_matrix(w: np.ndarray, scale: np.ndarray | None, fmt: int, act: int, K: int, N: int,
                  gs: int, e: int) -> np.ndarray:
    """Matrix e of a weight stack, converted or dequantised exactly to float64 [K][N]."""
    w = np.ascontiguousarray(w)
    scale = None if scale is None else np.ascontiguousarray(scale, dtype=np.uint16)
    out = np.empty((K, N), np.float64)
    lib().orc_expand_matrix(_p(w), _p(scale), fmt, act, K, N, gs, e, _p(out))
    return out


def layer(inputs: dict, cfg, ids: np.ndarray, w: np.ndarray, tokens=None, threads: int = 1) -> np.ndarray:
    """Layer output (float64 [len(tokens)][H]) for the given tokens (default: all), using
    routing (ids, w).  `threads` > 1 splits the token list into contiguous ranges run in
    parallel (rows are independent, so the result does not depend on the split)."""
    T, H = cfg.T, cfg.H
    tokens = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    keep = [inputs["x"], ids, w]
    a = _LayerArgs()
    a.T, a.H, a.I, a.k = T, H, cfg.I, cfg.k
    a.e_first, a.e_local = cfg.e_first, cfg.e_local
    a.act = BF16 if cfg.act == "bf16" else F32
    a.wfmt = {"int4": INT4, "fp8": FP8}.get(cfg.wfmt, DENSE)
    a.group_size = cfg.group_size
    a.shared_I = cfg.shared_I
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    keep += [ids, w]
    a.x, a.ids, a.w = _p(inputs["x"]), _p(ids), _p(w)
    for f, name in (("wg", "w_gate"), ("wu", "w_up"), ("wd", "w_down")):
        arr = np.ascontiguousarray(inputs[name])
        keep.append(arr)
        setattr(a, f, _p(arr))
    if cfg.wfmt in ("int4", "fp8"):
        for f, name in (("sg", "w_gate_scale"), ("su", "w_up_scale"), ("sd", "w_down_scale")):
            arr = np.ascontiguousarray(inputs[name], dtype=np.uint16)
            keep.append(arr)
            setattr(a, f, _p(arr))
    if cfg.shared_I:
        for f, name in (("shg", "shared_gate"), ("shu", "shared_up"), ("shd", "shared_down")):
            arr = np.ascontiguousarray(inputs[name])
            keep.append(arr)
            setattr(a, f, _p(arr))
    y = np.empty((len(tokens), H), np.float64)
    L = lib()
    if threads <= 1 or len(tokens) < 2:
        L.orc_layer(ctypes.byref(a), _p(tokens), len(tokens), _p(y))
    else:
        bounds = np.linspace(0, len(tokens), min(threads, len(tokens)) + 1).astype(int)

        def run(i):
            lo, hi = bounds[i], bounds[i + 1]
            if hi > lo:
                L.orc_layer(ctypes.byref(a), tokens[lo:].ctypes.data, int(hi - lo),
                            y[lo:].ctypes.data)

        with ThreadPoolExecutor(len(bounds) - 1) as ex:
            list(ex.map(run, range(len(bounds) - 1)))
    del keep
    return y
