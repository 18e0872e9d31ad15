"""The five entry points of the C ABI on torch tensors.

PyTorch is used only for device memory and the current stream: each function checks shapes,
dtypes and devices, then passes raw pointers to libmoe_mi355x.so.  Every step of the layer runs
in the library's HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes

import torch

from . import _abi
from ._abi import check, load

_DT = {torch.float32: _abi.MOE_DT_F32, torch.bfloat16: _abi.MOE_DT_BF16, torch.float16: _abi.MOE_DT_F16}


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("expected a GPU tensor")
            if not t.is_contiguous():
                raise ValueError("expected a contiguous tensor")


def _ptr(t):
    return None if t is None else t.data_ptr()


def route(logits: torch.Tensor, k: int, ids: torch.Tensor | None = None, w: torch.Tensor | None = None,
          stream=None):
    """Softmax top-k routing of fp32 logits [T][E] -> (ids int32 [T][k], w fp32 [T][k])."""
    T, E = logits.shape
    assert logits.dtype == torch.float32
    ids = ids if ids is not None else torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = w if w is not None else torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _dev(logits, ids, w)
    check("moe_route", load().moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream)))
    return ids, w


def pack_routing(ids: torch.Tensor, w: torch.Tensor, blob: torch.Tensor | None = None, stream=None):
    """ids int32 [T][k], w fp32 [T][k] -> blob int32 [2][T][k]."""
    T, k = ids.shape
    assert ids.dtype == torch.int32 and w.dtype == torch.float32 and w.shape == ids.shape
    blob = blob if blob is not None else torch.empty((2, T, k), dtype=torch.int32, device=ids.device)
    _dev(ids, w, blob)
    check("moe_pack_routing", load().moe_pack_routing(_ptr(ids), _ptr(w), T, k, _ptr(blob), _stream(stream)))
    return blob


def route_packed(logits: torch.Tensor, k: int, ids: torch.Tensor | None = None, w: torch.Tensor | None = None,
                 blob: torch.Tensor | None = None, write_ids: bool = True, stream=None):
    """route + pack_routing in one launch -> (ids, w, blob); ids and w are None when write_ids is
    False."""
    T, E = logits.shape
    assert logits.dtype == torch.float32
    dev = logits.device
    if write_ids:
        ids = ids if ids is not None else torch.empty((T, k), dtype=torch.int32, device=dev)
        w = w if w is not None else torch.empty((T, k), dtype=torch.float32, device=dev)
    else:
        ids = w = None
    blob = blob if blob is not None else torch.empty((2, T, k), dtype=torch.int32, device=dev)
    _dev(logits, ids, w, blob)
    check("moe_route_packed", load().moe_route_packed(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _ptr(blob),
                                                      _stream(stream)))
    return ids, w, blob


def prepare_router_weights(wr: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Router weight W_r fp32 [H][E] -> bf16 [2][E][H] (hi, lo planes) for router_logits."""
    H, E = wr.shape
    assert wr.dtype == torch.float32 and wr.is_contiguous()
    out = out if out is not None else torch.empty((2, E, H), dtype=torch.bfloat16, device=wr.device)
    _dev(wr, out)
    check("moe_prepare_router_weights", load().moe_prepare_router_weights(_ptr(wr), H, E, _ptr(out), _stream(stream)))
    return out


def router_logits(x: torch.Tensor, w_split: torch.Tensor, bias: torch.Tensor | None = None,
                  logits: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """x [T][H] (bf16 or fp32) -> fp32 logits [T][E] = x W_r (+ bias)."""
    T, H = x.shape
    E = w_split.shape[1]
    assert w_split.shape == (2, E, H) and w_split.dtype == torch.bfloat16
    logits = logits if logits is not None else torch.empty((T, E), dtype=torch.float32, device=x.device)
    _dev(x, w_split, bias, logits)
    check("moe_router_logits", load().moe_router_logits(_ptr(x), _DT[x.dtype], _ptr(w_split), _ptr(bias), T, H, E,
                                                        _ptr(logits), _stream(stream)))
    return logits


def route_hidden(x: torch.Tensor, w_split: torch.Tensor, k: int, bias: torch.Tensor | None = None,
                 logits=None, ids=None, w=None, blob=None, write_ids: bool = True, stream=None):
    """Router projection then route_packed -> (logits, ids, w, blob)."""
    T, H = x.shape
    E = w_split.shape[1]
    dev = x.device
    logits = logits if logits is not None else torch.empty((T, E), dtype=torch.float32, device=dev)
    if write_ids:
        ids = ids if ids is not None else torch.empty((T, k), dtype=torch.int32, device=dev)
        w = w if w is not None else torch.empty((T, k), dtype=torch.float32, device=dev)
    else:
        ids = w = None
    blob = blob if blob is not None else torch.empty((2, T, k), dtype=torch.int32, device=dev)
    _dev(x, w_split, bias, logits, ids, w, blob)
    check("moe_route_hidden", load().moe_route_hidden(_ptr(x), _DT[x.dtype], _ptr(w_split), _ptr(bias), T, H, E, k,
                                                      _ptr(logits), _ptr(ids), _ptr(w), _ptr(blob), _stream(stream)))
    return logits, ids, w, blob


def permute_workspace_bytes(T: int, k: int, e_local: int) -> int:
    return int(load().moe_permute_workspace_bytes(T, k, e_local))


def permute(blob: torch.Tensor, e_first: int, e_local: int, sorted_pairs=None, group_offsets=None,
            pair_pos=None, workspace=None, stream=None):
    """blob [2][T][k] -> (sorted_pairs [T*k], group_offsets [e_local+1], pair_pos [T*k])."""
    _, T, k = blob.shape
    assert blob.dtype == torch.int32
    dev = blob.device
    ws_bytes = permute_workspace_bytes(T, k, e_local)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    sp = sorted_pairs if sorted_pairs is not None else torch.empty(T * k, dtype=torch.int32, device=dev)
    off = group_offsets if group_offsets is not None else torch.empty(e_local + 1, dtype=torch.int32, device=dev)
    pp = pair_pos if pair_pos is not None else torch.empty(T * k, dtype=torch.int32, device=dev)
    _dev(blob, sp, off, pp, workspace)
    check("moe_permute", load().moe_permute(_ptr(blob), T, k, e_first, e_local, _ptr(sp), _ptr(off),
                                            _ptr(pp), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream)))
    return sp, off, pp


def permute_noalloc(blob: torch.Tensor, e_first: int, e_local: int, sorted_pairs: torch.Tensor,
                    group_offsets: torch.Tensor, pair_pos: torch.Tensor, stream=None):
    """permute() without a workspace, for callers that cannot allocate: the library keeps the
    per-chunk counts in its own fixed device array (moe_permute_noalloc).  The output tensors are
    the caller's; nothing is allocated here."""
    _, T, k = blob.shape
    assert blob.dtype == torch.int32
    _dev(blob, sorted_pairs, group_offsets, pair_pos)
    assert sorted_pairs.numel() >= T * k and pair_pos.numel() >= T * k and group_offsets.numel() >= e_local + 1
    check("moe_permute_noalloc", load().moe_permute_noalloc(_ptr(blob), T, k, e_first, e_local, _ptr(sorted_pairs),
                                                            _ptr(group_offsets), _ptr(pair_pos), _stream(stream)))
    return sorted_pairs, group_offsets, pair_pos


def prepare_dense_weights(w: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Dense weights [E][K][N] (x @ W) -> the same values stored [E][N][K] (MOE_W_DENSE_NK), the
    layout the bf16 grouped GEMM reads.  A one-time preparation, run by the library."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    E, K, N = w3.shape
    assert w3.is_contiguous() and w3.dtype in _DT
    out = out if out is not None else torch.empty((E, N, K), dtype=w.dtype, device=w.device)
    _dev(w3, out)
    check("moe_prepare_dense_weights", load().moe_prepare_dense_weights(_ptr(w3), E, K, N, _DT[w.dtype], _ptr(out),
                                                                        _stream(stream)))
    return out[0] if squeeze else out


def prepare_dense_weights_f16(w: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """bf16 dense weights [E][K][N] -> fp16 [E][N][K] holding 2^8 * w (MOE_W_DENSE_NK_F16), the
    weights of a down projection over fp16 h.  A one-time preparation, run by the library."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    E, K, N = w3.shape
    assert w3.is_contiguous() and w3.dtype == torch.bfloat16
    out = out if out is not None else torch.empty((E, N, K), dtype=torch.float16, device=w.device)
    assert out.dtype == torch.float16 and tuple(out.shape) == (E, N, K)
    _dev(w3, out)
    check("moe_prepare_dense_weights_f16", load().moe_prepare_dense_weights_f16(_ptr(w3), E, K, N, _ptr(out),
                                                                                _stream(stream)))
    return out[0] if squeeze else out


def grouped_gemm(op: int, a: torch.Tensor, group_offsets: torch.Tensor, w0: torch.Tensor,
                 w1: torch.Tensor | None, out: torch.Tensor, *, K: int, N: int, row_index=None,
                 row_div: int = 1, s0=None, s1=None, group_size: int = 0, m_hint: int = 0,
                 weights_nk: bool = True, stream=None):
    """One grouped GEMM (see moe_grouped_gemm in include/moe.h).  Dense weights are
    [n_groups][N][K] (weights_nk, from prepare_dense_weights) or [n_groups][K][N] (fp32 only) in the
    activation dtype, or fp16 [n_groups][N][K] from prepare_dense_weights_f16 (down projection over
    fp16 h); int4 weights are int32 words [n_groups][K/8][N] with bf16 scales s0/s1
    [n_groups][K/group_size][N]; fp8 (e4m3) weights are uint8 [n_groups][N][K] with bf16 scales
    s0/s1 [n_groups][N]."""
    _dev(a, group_offsets, w0, w1, out, row_index, s0, s1)
    args = _abi.MoeGemmArgs()
    args.op = op
    args.act_dtype = _DT[a.dtype]
    if w0.dtype == torch.int32:
        args.wfmt = _abi.MOE_W_INT4_SYM_GROUP
    elif w0.dtype == torch.uint8:
        args.wfmt = _abi.MOE_W_FP8_E4M3
    elif w0.dtype == torch.float16:
        args.wfmt = _abi.MOE_W_DENSE_NK_F16
    else:
        args.wfmt = _abi.MOE_W_DENSE_NK if weights_nk else _abi.MOE_W_DENSE
    args.group_size = {_abi.MOE_W_INT4_SYM_GROUP: group_size, _abi.MOE_W_FP8_E4M3: K}.get(args.wfmt, 0)
    args.K, args.N = K, N
    args.n_groups = group_offsets.numel() - 1
    args.rows_cap = out.shape[0]
    args.a_rows = a.shape[0]
    args.row_div = row_div
    args.m_hint = m_hint
    args.out_dtype = _DT[out.dtype]
    assert a.shape[1] == K and out.shape[1] == N
    args.a, args.row_index, args.group_offsets = _ptr(a), _ptr(row_index), _ptr(group_offsets)
    args.w0, args.w1, args.s0, args.s1, args.out = _ptr(w0), _ptr(w1), _ptr(s0), _ptr(s1), _ptr(out)
    check("moe_grouped_gemm", load().moe_grouped_gemm(ctypes.byref(args), _stream(stream)))
    return out


def combine(expert_out: torch.Tensor, blob: torch.Tensor, pair_pos: torch.Tensor, shared_out=None,
            y: torch.Tensor | None = None, y_dtype=None, stream=None):
    """-> y [T][H]: sum over each token's local slots of w * expert_out[row] (+ shared_out)."""
    _, T, k = blob.shape
    H = expert_out.shape[1]
    y_dtype = y_dtype or expert_out.dtype
    y = y if y is not None else torch.empty((T, H), dtype=y_dtype, device=expert_out.device)
    _dev(expert_out, blob, pair_pos, shared_out, y)
    if shared_out is not None:
        assert shared_out.dtype == expert_out.dtype and tuple(shared_out.shape) == (T, H)
    check("moe_combine", load().moe_combine(_ptr(expert_out), expert_out.shape[0], _DT[expert_out.dtype],
                                            _ptr(blob), _ptr(pair_pos), _ptr(shared_out), T, k, H, _ptr(y),
                                            _DT[y.dtype], _stream(stream)))
    return y
