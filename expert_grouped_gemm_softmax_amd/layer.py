"""One device's share of a routed MoE feed-forward layer, composed from the C ABI's five calls:
route -> pack_routing -> permute -> grouped_gemm(gate/up + SwiGLU) -> grouped_gemm(down)
[-> shared expert] -> combine.  Buffers are allocated once per token count and reused."""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import _abi, ops


@dataclass
class ExpertWeights:
    """Device-resident weights of the local experts (and of the optional shared expert).

    A layer weight W is K x N (output n = sum_k a[k] W[k][n]); K = H, N = I for gate/up and the
    reverse for down.  Dense weights are held prepared, [e_local][N][K] (written by the library
    from the stated [e_local][K][N]; see upload): w_gate, w_up [e_local][I][H] in the activation
    dtype, w_down [e_local][H][I] in the dtype of the SwiGLU output h (fp16 holding 2^8 * W by
    default, or bf16); shared expert gate, up [Is][H], down [H][Is] likewise.
    int4: int32 words [e_local][K/8][N] plus bf16 scales [e_local][K/group_size][N] (group_size 0:
    channel-wise, one scale per column over all K); h is fp16.  fp8: e4m3 bytes [e_local][N][K]
    plus bf16 scales [e_local][N]; h fp16 (or bf16)."""
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    s_gate: torch.Tensor | None = None
    s_up: torch.Tensor | None = None
    s_down: torch.Tensor | None = None
    group_size: int = 0
    shared_gate: torch.Tensor | None = None
    shared_up: torch.Tensor | None = None
    shared_down: torch.Tensor | None = None

    h_fp8: torch.dtype = torch.float16   # h's dtype over fp8 down weights (fp16 or bf16)
    stated_layout: bool = False          # dense bf16 weights left [e][K][N] (no preparation)

    @property
    def int4(self) -> bool:
        return self.w_gate.dtype == torch.int32

    @property
    def fp8(self) -> bool:
        return self.w_gate.dtype == torch.uint8

    @property
    def h_dtype(self) -> torch.dtype:
        """dtype of the SwiGLU output h between the two GEMMs: fp16 over fp16 or int4 down weights
        (the fp16 MFMA path), either 16-bit type over fp8 ones, else the down weights' dtype."""
        if self.int4:
            return torch.float16
        return self.h_fp8 if self.fp8 else self.w_down.dtype


# Measured on one MI355X (bench.py, paired workloads with the same routing): W4A16 over bf16
# expert weights, step time ratio bf16 / W4A16 -- 1.7-1.8 at 10 rows per expert (decode), 1.07 at
# 160 (prefill), 0.81 under the skewed routing (1280 rows per expert, hot experts of 8192): int4
# pays where the expert weights are streamed (fewer bytes), bf16 where the matrix units bind (its
# prefill tiles copy operands straight to LDS, int4 dequantises through registers).
W4A16_MAX_ROWS_PER_EXPERT = 192


def choose_weight_format(rows_per_expert: float) -> str:
    """Weight format for the routed experts by the expected rows per expert (T * k / E): "int4"
    (W4A16) up to W4A16_MAX_ROWS_PER_EXPERT rows, where this library measured it at least as fast
    as bf16, else "bf16".  The layer's accuracy is the same either way (both meet the parity bar)."""
    return "int4" if rows_per_expert <= W4A16_MAX_ROWS_PER_EXPERT else "bf16"


def _t(a: np.ndarray, device) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns, uint8 arrays fp8 bytes."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload(inputs: dict, cfg, device="cuda", h_dtype=torch.float16,
           stated_layout: bool = False) -> tuple[torch.Tensor, torch.Tensor, ExpertWeights]:
    """Copy a workloads.make_inputs() dict to the GPU -> (x, logits, weights).  Dense weights
    arrive [E][K][N] and are prepared once by the library: gate/up with moe_prepare_dense_weights,
    the down projections of a bf16 layer with moe_prepare_dense_weights_f16 when h_dtype is fp16
    (the default: h rounded to fp16, 8x finer than bf16) or moe_prepare_dense_weights for bf16 h."""
    x = _t(inputs["x"], device)
    logits = _t(inputs["logits"], device)
    assert h_dtype in (torch.float16, torch.bfloat16)
    if stated_layout:
        # dense bf16 weights as the layer states them, [e][K][N] (MOE_W_DENSE): the grouped GEMM
        # reads their K rows and transposes its operands; h is bf16 (down weights stay bf16)
        assert cfg.wfmt == "dense" and cfg.act == "bf16" and not cfg.shared_I
        return x, logits, ExpertWeights(w_gate=_t(inputs["w_gate"], device), w_up=_t(inputs["w_up"], device),
                                        w_down=_t(inputs["w_down"], device), stated_layout=True)

    def dense(name):
        return ops.prepare_dense_weights(_t(inputs[name], device))

    def dense_down(name):
        w = _t(inputs[name], device)
        if w.dtype == torch.bfloat16 and h_dtype == torch.float16:
            return ops.prepare_dense_weights_f16(w)
        return ops.prepare_dense_weights(w)

    if cfg.wfmt in ("int4", "fp8"):
        kw = dict(w_gate=_t(inputs["w_gate"], device), w_up=_t(inputs["w_up"], device),
                  w_down=_t(inputs["w_down"], device),
                  s_gate=_t(inputs["w_gate_scale"], device), s_up=_t(inputs["w_up_scale"], device),
                  s_down=_t(inputs["w_down_scale"], device),
                  group_size=cfg.group_size if cfg.wfmt == "int4" else 0, h_fp8=h_dtype)
    else:
        kw = dict(w_gate=dense("w_gate"), w_up=dense("w_up"), w_down=dense_down("w_down"))
    if cfg.shared_I:
        kw.update(shared_gate=dense("shared_gate"), shared_up=dense("shared_up"),
                  shared_down=dense_down("shared_down"))
    return x, logits, ExpertWeights(**kw)


@dataclass
class Buffers:
    ids: torch.Tensor
    w: torch.Tensor
    blob: torch.Tensor
    sorted_pairs: torch.Tensor
    group_offsets: torch.Tensor
    pair_pos: torch.Tensor
    h: torch.Tensor
    o: torch.Tensor
    y: torch.Tensor
    workspace: torch.Tensor | None = None
    shared_offsets: torch.Tensor | None = None
    shared_h: torch.Tensor | None = None
    shared_o: torch.Tensor | None = None
    extra: dict = field(default_factory=dict)


class MoELayer:
    """Routed MoE layer over local experts [e_first, e_first + e_local) of E global experts."""

    def __init__(self, H: int, I: int, E: int, k: int, e_first: int, e_local: int,
                 weights: ExpertWeights, act_dtype=torch.bfloat16, y_dtype=torch.float32):
        self.H, self.I, self.E, self.k = H, I, E, k
        self.e_first, self.e_local = e_first, e_local
        self.weights = weights
        self.act_dtype = act_dtype
        # The layer output is fp32 (a partial sum, over devices in an expert-parallel
        # reduce-scatter).  Expert output rows take h's dtype when that is fp16 (its 2^-12 rounding
        # is small beside the bar, and the combine reads half the bytes; it accumulates in fp32),
        # else fp32: a bf16 rounding of every row would add an error proportional to |y|.
        self.y_dtype = y_dtype
        self.h_dtype = weights.h_dtype if act_dtype == torch.bfloat16 else act_dtype
        self.o_dtype = torch.float16 if self.h_dtype == torch.float16 else torch.float32
        self.shared_I = 0 if weights.shared_gate is None else weights.shared_gate.shape[0]
        self._check_shapes()
        self._buf: dict[int, Buffers] = {}

    def _check_shapes(self):
        W, H, I, el = self.weights, self.H, self.I, self.e_local
        if W.shared_down is not None and not W.int4 and W.shared_down.dtype != W.w_down.dtype:
            raise ValueError("shared and routed down projections need one h dtype")
        if W.int4 and W.shared_down is not None and W.shared_down.dtype != torch.float16:
            raise ValueError("an int4 layer's shared down projection reads fp16 h: prepare it with "
                             "prepare_dense_weights_f16")
        if W.int4:
            want = {"w_gate": (el, H // 8, I), "w_up": (el, H // 8, I), "w_down": (el, I // 8, H)}
        elif W.stated_layout:
            want = {"w_gate": (el, H, I), "w_up": (el, H, I), "w_down": (el, I, H)}
        elif W.fp8:
            want = {"w_gate": (el, I, H), "w_up": (el, I, H), "w_down": (el, H, I),
                    "s_gate": (el, I), "s_up": (el, I), "s_down": (el, H)}
        else:
            want = {"w_gate": (el, I, H), "w_up": (el, I, H), "w_down": (el, H, I)}
        if self.shared_I:
            Is = self.shared_I
            want.update(shared_gate=(Is, H), shared_up=(Is, H), shared_down=(H, Is))
        for name, shape in want.items():
            got = tuple(getattr(W, name).shape)
            if got != shape:
                raise ValueError(f"{name}: shape {got}, expected {shape}")

    @classmethod
    def from_config(cls, cfg, weights: ExpertWeights, y_dtype=torch.float32):
        act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
        return cls(cfg.H, cfg.I, cfg.E, cfg.k, cfg.e_first, cfg.e_local, weights, act, y_dtype)

    def rows_capacity(self, T: int) -> int:
        return T * min(self.k, self.e_local)

    def buffers(self, T: int, device) -> Buffers:
        b = self._buf.get(T)
        if b is None:
            k, cap = self.k, self.rows_capacity(T)
            i32 = dict(dtype=torch.int32, device=device)
            b = Buffers(ids=torch.empty((T, k), **i32), w=torch.empty((T, k), dtype=torch.float32, device=device),
                        blob=torch.empty((2, T, k), **i32), sorted_pairs=torch.empty(T * k, **i32),
                        group_offsets=torch.empty(self.e_local + 1, **i32), pair_pos=torch.empty(T * k, **i32),
                        h=torch.empty((cap, self.I), dtype=self.h_dtype, device=device),
                        o=torch.empty((cap, self.H), dtype=self.o_dtype, device=device),
                        y=torch.empty((T, self.H), dtype=self.y_dtype, device=device))
            b.workspace = torch.empty(max(1, ops.permute_workspace_bytes(T, k, self.e_local)),
                                      dtype=torch.uint8, device=device)
            if self.shared_I:
                b.shared_offsets = torch.tensor([0, T], **i32)
                b.shared_h = torch.empty((T, self.shared_I), dtype=self.h_dtype, device=device)
                b.shared_o = torch.empty((T, self.H), dtype=self.o_dtype, device=device)
            self._buf[T] = b
        return b

    def m_hint(self, T: int) -> int:
        return max(1, -(-T * self.k // self.E))

    # -- the steps, individually callable (the benchmark times them one by one) -----------------
    def step_route(self, logits, b, stream=None):
        ops.route_packed(logits, self.k, b.ids, b.w, b.blob, stream=stream)
        ops.permute(b.blob, self.e_first, self.e_local, b.sorted_pairs, b.group_offsets, b.pair_pos,
                    workspace=b.workspace, stream=stream)

    def step_gate_up(self, x, b, stream=None):
        W = self.weights
        ops.grouped_gemm(_abi.MOE_OP_GATE_UP_SWIGLU, x, b.group_offsets, W.w_gate, W.w_up, b.h,
                         K=self.H, N=self.I, row_index=b.sorted_pairs, row_div=self.k, s0=W.s_gate,
                         s1=W.s_up, group_size=W.group_size or self.H, m_hint=self.m_hint(x.shape[0]),
                         weights_nk=not W.stated_layout, stream=stream)

    def step_down(self, x, b, stream=None):
        W = self.weights
        ops.grouped_gemm(_abi.MOE_OP_DOWN, b.h, b.group_offsets, W.w_down, None, b.o, K=self.I, N=self.H,
                         s0=W.s_down, group_size=W.group_size or self.I, m_hint=self.m_hint(x.shape[0]),
                         weights_nk=not W.stated_layout, stream=stream)

    def step_shared(self, x, b, stream=None):
        W, T = self.weights, x.shape[0]
        ops.grouped_gemm(_abi.MOE_OP_GATE_UP_SWIGLU, x, b.shared_offsets, W.shared_gate, W.shared_up,
                         b.shared_h, K=self.H, N=self.shared_I, m_hint=T, stream=stream)
        ops.grouped_gemm(_abi.MOE_OP_DOWN, b.shared_h, b.shared_offsets, W.shared_down, None, b.shared_o,
                         K=self.shared_I, N=self.H, m_hint=T, stream=stream)

    def step_combine(self, b, stream=None):
        ops.combine(b.o, b.blob, b.pair_pos, b.shared_o if self.shared_I else None, b.y, stream=stream)

    def forward(self, x: torch.Tensor, logits: torch.Tensor, stream=None) -> torch.Tensor:
        """x [T][H] (activation dtype), logits fp32 [T][E] -> y [T][H] (y dtype).  The returned
        tensor is this layer's buffer for T tokens and is overwritten by the next call."""
        T = x.shape[0]
        assert x.dtype == self.act_dtype and tuple(logits.shape) == (T, self.E)
        b = self.buffers(T, x.device)
        if stream is None:                        # looked up once: each lookup costs microseconds
            stream = torch.cuda.current_stream()
        self.step_route(logits, b, stream)
        self.step_gate_up(x, b, stream)
        self.step_down(x, b, stream)
        if self.shared_I:
            self.step_shared(x, b, stream)
        self.step_combine(b, stream)
        return b.y
