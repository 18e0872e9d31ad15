"""The C-ABI library on the CPU: it loads, exports every symbol include/moe.h declares, and
rejects invalid arguments before any HIP call (so nothing here needs a GPU)."""
import ctypes
import os
import subprocess

import pytest

from expert_grouped_gemm_softmax_amd import _abi
from expert_grouped_gemm_softmax_amd._abi import MoeGemmArgs

INV, UNS = _abi.MOE_ERR_INVALID_ARG, _abi.MOE_ERR_UNSUPPORTED
FAKE = 0x1000  # never dereferenced: validation rejects these calls first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_abi.LIB_PATH):
        pytest.fail("libmoe_mi355x.so is not built (run __graft_entry__.build())")
    return _abi.load()


def test_exports_every_declared_symbol(L):
    declared = _abi.header_functions()
    assert set(declared) >= {"moe_route", "moe_pack_routing", "moe_permute", "moe_grouped_gemm",
                             "moe_combine", "moe_status_string", "moe_abi_version"}
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared) <= exported
    # only the C ABI is exported
    assert {s for s in exported if not s.startswith("moe_")} <= {"_init", "_fini"}


def test_version_and_status_strings(L):
    assert L.moe_abi_version() == 2
    for s in range(5):
        assert L.moe_status_string(s)
    assert b"scratch" in L.moe_status_string(_abi.MOE_ERR_SCRATCH_TOO_SMALL)
    assert L.moe_status_string(99) == b"unknown status"


def test_gfx950_code_object_only():
    import re
    with open(_abi.LIB_PATH, "rb") as f:
        data = f.read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-f]+)", data))
    assert targets == {b"gfx950"}, targets


def test_route_validation(L):
    ok = (FAKE, 8, 16, 2, FAKE, FAKE, None)
    bad = [
        (None, 8, 16, 2, FAKE, FAKE, None), (FAKE, 8, 16, 2, None, FAKE, None),
        (FAKE, 8, 16, 2, FAKE, None, None), (FAKE, 0, 16, 2, FAKE, FAKE, None),
        (FAKE, 8, 0, 1, FAKE, FAKE, None), (FAKE, 8, 1025, 2, FAKE, FAKE, None),
        (FAKE, 8, 16, 0, FAKE, FAKE, None), (FAKE, 8, 16, 17, FAKE, FAKE, None),
        (FAKE, 8, 512, 65, FAKE, FAKE, None), (FAKE, 1 << 22, 1024, 2, FAKE, FAKE, None),
    ]
    for args in bad:
        assert L.moe_route(*args) == INV, args
    assert ok  # the valid form would launch; not called without a GPU


def test_route_packed_validation(L):
    bad = [
        (None, 8, 16, 2, FAKE, FAKE, FAKE, None), (FAKE, 8, 16, 2, FAKE, FAKE, None, None),
        (FAKE, 8, 16, 2, None, FAKE, FAKE, None), (FAKE, 8, 16, 2, FAKE, None, FAKE, None),
        (FAKE, 0, 16, 2, FAKE, FAKE, FAKE, None), (FAKE, 8, 1025, 2, FAKE, FAKE, FAKE, None),
        (FAKE, 8, 16, 0, None, None, FAKE, None), (FAKE, 8, 16, 17, None, None, FAKE, None),
        (FAKE, 8, 512, 65, FAKE, FAKE, FAKE, None), (FAKE, 1 << 22, 1024, 2, None, None, FAKE, None),
    ]
    for args in bad:
        assert L.moe_route_packed(*args) == INV, args


def test_pack_and_permute_validation(L):
    assert L.moe_pack_routing(None, FAKE, 4, 2, FAKE, None) == INV
    assert L.moe_pack_routing(FAKE, FAKE, 4, 65, FAKE, None) == INV
    assert L.moe_pack_routing(FAKE, FAKE, 0, 2, FAKE, None) == INV
    assert L.moe_pack_routing(FAKE, FAKE, 1 << 26, 64, FAKE, None) == INV
    assert L.moe_permute_workspace_bytes(4, 2, 8) == 0    # one workgroup: no workspace
    assert L.moe_permute_workspace_bytes(2048, 8, 64) == 0  # 16384 pairs: still one workgroup
    ws = L.moe_permute_workspace_bytes(2049, 8, 8)
    assert ws == 33 * 8 * 4                               # 33 chunks of 512 pairs, per-expert counts
    assert L.moe_permute_workspace_bytes(8192, 10, 64) == 160 * 64 * 4
    assert L.moe_permute_workspace_bytes(0, 2, 8) == 0
    assert L.moe_permute(None, 2049, 8, 0, 8, FAKE, FAKE, FAKE, FAKE, ws, None) == INV
    assert L.moe_permute(FAKE, 2049, 8, 0, 8, FAKE, None, FAKE, FAKE, ws, None) == INV
    assert L.moe_permute(FAKE, 2049, 8, 0, 0, FAKE, FAKE, FAKE, FAKE, ws, None) == INV
    assert L.moe_permute(FAKE, 2049, 8, 0, 1025, FAKE, FAKE, FAKE, FAKE, ws, None) == INV
    assert L.moe_permute(FAKE, 2049, 8, -1, 8, FAKE, FAKE, FAKE, FAKE, ws, None) == INV
    assert L.moe_permute(FAKE, 2049, 0, 0, 8, FAKE, FAKE, FAKE, FAKE, ws, None) == INV
    assert L.moe_permute(FAKE, 2049, 8, 0, 8, FAKE, FAKE, FAKE, None, ws, None) == INV
    assert L.moe_permute(FAKE, 2049, 8, 0, 8, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == INV
    assert L.moe_permute(FAKE, 2049, 8, 0, 8, FAKE, FAKE, FAKE, FAKE + 4, ws, None) == INV   # alignment


def test_permute_noalloc_validation(L):
    """Host checks of the allocation-free permutation, including inputs whose per-chunk counts
    would not fit its fixed scratch array (all rejected before any HIP call)."""
    F = FAKE
    TOO_BIG = _abi.MOE_ERR_SCRATCH_TOO_SMALL
    assert L.moe_permute_noalloc(None, 2049, 8, 0, 8, F, F, F, None) == INV
    assert L.moe_permute_noalloc(F, 2049, 8, 0, 8, None, F, F, None) == INV
    assert L.moe_permute_noalloc(F, 2049, 8, 0, 8, F, None, F, None) == INV
    assert L.moe_permute_noalloc(F, 2049, 8, 0, 8, F, F, None, None) == INV
    assert L.moe_permute_noalloc(F, 0, 8, 0, 8, F, F, F, None) == INV
    assert L.moe_permute_noalloc(F, 2049, 65, 0, 8, F, F, F, None) == INV
    assert L.moe_permute_noalloc(F, 2049, 8, -1, 8, F, F, F, None) == INV
    assert L.moe_permute_noalloc(F, 2049, 8, 0, 1025, F, F, F, None) == INV
    cap = _abi.MOE_PERMUTE_NOALLOC_SCRATCH_BYTES
    # 1024 local experts: 1024 chunks of 512 pairs fit exactly, one more chunk does not
    assert L.moe_permute_workspace_bytes(1024 * 512 // 64, 64, 1024) == cap
    assert L.moe_permute_noalloc(F, 1024 * 512 // 64 + 8, 64, 0, 1024, F, F, F, None) == TOO_BIG
    assert L.moe_permute_noalloc(F, (1 << 23) // 64 + 8, 64, 0, 64, F, F, F, None) == TOO_BIG


def _gemm(**kw):
    a = MoeGemmArgs()
    base = dict(op=0, act_dtype=1, wfmt=2, group_size=0, K=256, N=128, n_groups=8, rows_cap=64,
                a_rows=32, row_div=2, m_hint=0, out_dtype=1, a=FAKE, row_index=FAKE, group_offsets=FAKE,
                w0=FAKE, w1=FAKE, s0=None, s1=None, out=FAKE)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(op=2), INV), (dict(act_dtype=7), UNS), (dict(wfmt=5), UNS), (dict(out_dtype=0), INV),
    (dict(wfmt=0, act_dtype=1, out_dtype=0), INV),       # gate/up never writes fp32 from bf16
    (dict(out_dtype=4), UNS), (dict(act_dtype=0, out_dtype=1), INV),
    (dict(a=None), INV), (dict(group_offsets=None), INV), (dict(w0=None), INV), (dict(out=None), INV),
    (dict(w1=None), INV), (dict(op=1, K=128, N=256, w1=FAKE), INV), (dict(K=32), INV), (dict(K=96), INV),
    (dict(N=32), INV), (dict(N=96), INV), (dict(op=1, K=128, N=192, w1=None), INV),
    (dict(n_groups=0), INV), (dict(n_groups=1025), INV), (dict(rows_cap=0), INV), (dict(a_rows=0), INV),
    (dict(row_div=0), INV), (dict(m_hint=-1), INV), (dict(row_index=None, a_rows=10), INV),
    (dict(wfmt=1, act_dtype=0, out_dtype=0, group_size=128, s0=FAKE, s1=FAKE), UNS),
    (dict(wfmt=1, out_dtype=2, group_size=20, s0=FAKE, s1=FAKE), UNS),      # not whole words
    (dict(wfmt=1, out_dtype=2, group_size=4, s0=FAKE, s1=FAKE), UNS),
    (dict(wfmt=1, out_dtype=2, group_size=96, s0=FAKE, s1=FAKE), UNS),      # does not divide K
    (dict(wfmt=1, out_dtype=2, K=192, group_size=48, s0=FAKE, s1=FAKE), UNS),   # neither divides nor is a multiple of 64
    (dict(wfmt=1, out_dtype=2, K=192, group_size=128, s0=FAKE, s1=FAKE), UNS),
    # int4 runs on fp16 operands: gate/up writes fp16 h, down reads fp16 h
    (dict(wfmt=1, out_dtype=1, group_size=128, s0=FAKE, s1=FAKE), UNS),
    (dict(op=1, K=128, N=256, w1=None, wfmt=1, act_dtype=1, out_dtype=0, group_size=128, s0=FAKE), UNS),
    # fp16 h over fp16 weights, bf16 h over bf16 weights; no fp16 gate/up input
    (dict(op=1, K=128, N=256, w1=None, wfmt=3, act_dtype=1, out_dtype=0), UNS),
    (dict(op=1, K=128, N=256, w1=None, wfmt=2, act_dtype=2, out_dtype=0), UNS),
    (dict(op=1, K=128, N=256, w1=None, wfmt=0, act_dtype=2, out_dtype=0), UNS),   # [K][N] weights are bf16
    (dict(op=1, K=128, N=256, w1=None, wfmt=3, act_dtype=2, out_dtype=1), INV),
    (dict(act_dtype=2, out_dtype=2), UNS), (dict(wfmt=3, out_dtype=2), UNS),
    (dict(act_dtype=0, out_dtype=0, wfmt=3), UNS),
    # fp8: scales required (two for gate/up, one for down), one per output channel (group = K)
    (dict(wfmt=4, out_dtype=2, group_size=256), INV), (dict(wfmt=4, out_dtype=2, group_size=256, s0=FAKE), INV),
    (dict(op=1, K=128, N=256, w1=None, wfmt=4, act_dtype=2, out_dtype=0, group_size=128, s0=FAKE, s1=FAKE), INV),
    (dict(wfmt=4, out_dtype=2, group_size=128, s0=FAKE, s1=FAKE), UNS),
    (dict(wfmt=4, act_dtype=0, out_dtype=0, group_size=256, s0=FAKE, s1=FAKE), UNS),
    (dict(wfmt=4, act_dtype=2, out_dtype=2, group_size=256, s0=FAKE, s1=FAKE), UNS),
    (dict(wfmt=1, group_size=128, s0=None, s1=FAKE), INV),
    (dict(wfmt=1, group_size=128, s0=FAKE, s1=None), INV),
    (dict(group_size=128), INV), (dict(s0=FAKE), INV),
    # 32-bit offsets: activation bytes below 2^31, one expert matrix below 2^32
    (dict(a_rows=1 << 17, K=8192), UNS), (dict(act_dtype=0, out_dtype=0, a_rows=1 << 17, K=4096), UNS),
    (dict(K=65536, N=32768), UNS),
])
def test_grouped_gemm_validation(L, kw, code):
    assert L.moe_grouped_gemm(ctypes.byref(_gemm(**kw)), None) == code
    assert L.moe_grouped_gemm(None, None) == INV


def test_combine_validation(L):
    ok = [FAKE, 64, 1, FAKE, FAKE, None, 8, 2, 256, FAKE, 1, None]
    for i, v in [(0, None), (1, 0), (3, None), (4, None), (6, 0), (7, 0), (7, 65), (8, 0), (8, 12),
                 (9, None)]:
        args = list(ok)
        args[i] = v
        assert L.moe_combine(*args) == INV, (i, v)
    for i, v in [(2, 3), (10, 9), (10, 2)]:
        args = list(ok)
        args[i] = v
        assert L.moe_combine(*args) == UNS, (i, v)


def test_prepare_dense_weights_validation(L):
    F = FAKE
    assert L.moe_prepare_dense_weights(None, 2, 64, 64, 1, F, None) == INV
    assert L.moe_prepare_dense_weights(F, 2, 64, 64, 1, None, None) == INV
    assert L.moe_prepare_dense_weights(F, 2, 64, 64, 7, F, None) == UNS
    assert L.moe_prepare_dense_weights(F, 0, 64, 64, 1, F, None) == INV
    assert L.moe_prepare_dense_weights(F, 2, 0, 64, 1, F, None) == INV
    assert L.moe_prepare_dense_weights(F, 2, 64, 0, 1, F, None) == INV
    assert L.moe_prepare_dense_weights(F, 65536, 64, 64, 1, F, None) == INV
    assert L.moe_prepare_dense_weights(F, 1, (1 << 22) + 1, 64, 1, F, None) == INV
    assert L.moe_prepare_dense_weights(F, 1024, 1 << 15, 1 << 15, 1, F, None) == INV   # 2^40 elements


def test_prepare_dense_weights_f16_validation(L):
    F = FAKE
    assert L.moe_prepare_dense_weights_f16(None, 2, 64, 64, F, None) == INV
    assert L.moe_prepare_dense_weights_f16(F, 2, 64, 64, None, None) == INV
    assert L.moe_prepare_dense_weights_f16(F, 0, 64, 64, F, None) == INV
    assert L.moe_prepare_dense_weights_f16(F, 2, 0, 64, F, None) == INV
    assert L.moe_prepare_dense_weights_f16(F, 2, 64, 0, F, None) == INV
    assert L.moe_prepare_dense_weights_f16(F, 1024, 1 << 15, 1 << 15, F, None) == INV
    # the bf16 -> fp16 preparation has its own entry point
    assert L.moe_prepare_dense_weights(F, 2, 64, 64, 2, F, None) == UNS


def test_calibration_library_exports_and_rejects_bad_sizes():
    """The measured-ceiling microkernels used by bench.py (a separate library): symbols, the flop
    count of the MFMA loop, and argument checks that return before any HIP call."""
    from expert_grouped_gemm_softmax_amd import build as hip_build
    if not os.path.exists(hip_build.CALIB_PATH):
        pytest.fail("libmoe_calib.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(hip_build.CALIB_PATH)
    lib.moe_calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.moe_calib_mfma_flops.restype = ctypes.c_double
    assert lib.moe_calib_mfma_flops(2, 3) == 2 * 4 * 3 * 8 * 16 * 16 * 32 * 2
    lib.moe_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    HIP_INVALID = 1                                   # hipErrorInvalidValue
    assert lib.moe_calib_mfma(0, 10, FAKE, None) == HIP_INVALID
    assert lib.moe_calib_mfma(4, 0, FAKE, None) == HIP_INVALID
    assert lib.moe_calib_mfma(4, 10, None, None) == HIP_INVALID
    unit = 8 * 256 * 8 * 16
    assert lib.moe_calib_read(None, unit, 8, FAKE, None) == HIP_INVALID
    assert lib.moe_calib_read(FAKE, unit + 16, 8, FAKE, None) == HIP_INVALID
    assert lib.moe_calib_read(FAKE, unit, 8, None, None) == HIP_INVALID


def test_router_entry_points_validation(L):
    F = FAKE
    # moe_prepare_router_weights(wr, H, E, out, stream)
    assert L.moe_prepare_router_weights(None, 64, 8, F, None) == INV
    assert L.moe_prepare_router_weights(F, 64, 8, None, None) == INV
    assert L.moe_prepare_router_weights(F, 0, 8, F, None) == INV
    assert L.moe_prepare_router_weights(F, 64, 0, F, None) == INV
    assert L.moe_prepare_router_weights(F, 64, 1025, F, None) == INV
    # moe_router_logits(x, x_dtype, w_split, bias, T, H, E, logits, stream)
    assert L.moe_router_logits(None, 1, F, None, 8, 64, 16, F, None) == INV
    assert L.moe_router_logits(F, 1, None, None, 8, 64, 16, F, None) == INV
    assert L.moe_router_logits(F, 1, F, None, 8, 64, 16, None, None) == INV
    assert L.moe_router_logits(F, 2, F, None, 8, 64, 16, F, None) == UNS       # fp16 x
    assert L.moe_router_logits(F, 1, F, None, 0, 64, 16, F, None) == INV
    assert L.moe_router_logits(F, 1, F, None, 8, 64, 1025, F, None) == INV
    assert L.moe_router_logits(F, 1, F, None, 1 << 20, 1 << 12, 16, F, None) == INV   # x bytes >= 2^31
    # moe_route_hidden(x, x_dtype, w_split, bias, T, H, E, k, logits, ids, w, blob, stream)
    assert L.moe_route_hidden(F, 1, F, None, 8, 64, 16, 2, None, F, F, F, None) == INV
    assert L.moe_route_hidden(F, 1, F, None, 8, 64, 16, 2, F, F, F, None, None) == INV
    assert L.moe_route_hidden(F, 1, F, None, 8, 64, 16, 2, F, None, F, F, None) == INV
    assert L.moe_route_hidden(F, 1, F, None, 8, 64, 16, 0, F, F, F, F, None) == INV
    assert L.moe_route_hidden(F, 1, F, None, 8, 64, 16, 17, F, F, F, F, None) == INV
    assert L.moe_route_hidden(F, 0, F, None, 8, 64, 1025, 2, F, F, F, F, None) == INV


def test_misaligned_pointers_are_invalid(L):
    """Each pointer argument one alignment unit off (2 bytes for 4-byte arrays, 8 bytes for
    16-byte ones) is rejected before any HIP call; the aligned call differs only there."""
    F, A2, A8 = FAKE, FAKE + 2, FAKE + 8
    # moe_route(logits, T, E, k, ids, w, stream)
    for i in (0, 4, 5):
        args = [F, 8, 16, 2, F, F, None]
        args[i] = A2
        assert L.moe_route(*args) == INV, i
    # moe_route_packed(logits, T, E, k, ids, w, blob, stream)
    for i in (0, 4, 5, 6):
        args = [F, 8, 16, 2, F, F, F, None]
        args[i] = A2
        assert L.moe_route_packed(*args) == INV, i
    for i in (0, 1, 4):
        args = [F, F, 4, 2, F, None]
        args[i] = A2
        assert L.moe_pack_routing(*args) == INV, i
    ws = L.moe_permute_workspace_bytes(2049, 8, 8)
    for i in (0, 5, 6, 7):
        args = [F, 2049, 8, 0, 8, F, F, F, F, ws, None]
        args[i] = A2
        assert L.moe_permute(*args) == INV, i
        noalloc = [F, 2049, 8, 0, 8, F, F, F, None]
        noalloc[i] = A2
        assert L.moe_permute_noalloc(*noalloc) == INV, i
    for f in ("a", "w0", "w1", "out"):
        assert L.moe_grouped_gemm(ctypes.byref(_gemm(**{f: A8})), None) == INV, f
    for f in ("row_index", "group_offsets"):
        assert L.moe_grouped_gemm(ctypes.byref(_gemm(**{f: A2})), None) == INV, f
    q4 = dict(wfmt=1, out_dtype=2, group_size=128)
    assert L.moe_grouped_gemm(ctypes.byref(_gemm(s0=A8, s1=F, **q4)), None) == INV
    assert L.moe_grouped_gemm(ctypes.byref(_gemm(s0=F, s1=A8, **q4)), None) == INV
    # moe_combine(expert_out, rows, act, blob, pair_pos, shared_out, T, k, H, y, y_dtype, stream)
    for i, v in ((0, A8), (3, A2), (4, A2), (5, A8), (9, A8)):
        args = [F, 64, 1, F, F, None, 8, 2, 256, F, 1, None]
        args[i] = v
        assert L.moe_combine(*args) == INV, i
    assert L.moe_prepare_dense_weights(A8, 2, 64, 64, 1, F, None) == INV
    assert L.moe_prepare_dense_weights(F, 2, 64, 64, 1, A8, None) == INV
    assert L.moe_prepare_dense_weights_f16(A8, 2, 64, 64, F, None) == INV
    assert L.moe_prepare_dense_weights_f16(F, 2, 64, 64, A8, None) == INV
    assert L.moe_prepare_router_weights(A2, 64, 8, F, None) == INV
    assert L.moe_prepare_router_weights(F, 64, 8, A8, None) == INV
    for i, v in ((0, A8), (2, A8), (3, A2), (7, A2)):
        args = [F, 1, F, None, 8, 64, 16, F, None]
        args[i] = v
        assert L.moe_router_logits(*args) == INV, i
    for i, v in ((0, A8), (2, A8), (3, A2), (8, A2), (9, A2), (10, A2), (11, A2)):
        args = [F, 1, F, None, 8, 64, 16, 2, F, F, F, F, None]
        args[i] = v
        assert L.moe_route_hidden(*args) == INV, i


def test_weight_format_rule():
    """The bf16 / W4A16 choice by rows per expert (host logic): int4 where the expert weights are
    streamed (decode), bf16 where the matrix units bind (skewed hot experts)."""
    from expert_grouped_gemm_softmax_amd.layer import W4A16_MAX_ROWS_PER_EXPERT, choose_weight_format
    assert choose_weight_format(10) == "int4"          # decode: 512 tokens x 10 / 512 experts
    assert choose_weight_format(160) == "int4"         # prefill
    assert choose_weight_format(1280) == "bf16"        # skewed routing, T = 8192
    assert choose_weight_format(W4A16_MAX_ROWS_PER_EXPERT) == "int4"
    assert choose_weight_format(W4A16_MAX_ROWS_PER_EXPERT + 1) == "bf16"
