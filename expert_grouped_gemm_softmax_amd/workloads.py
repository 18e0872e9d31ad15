"""Seeded synthetic inputs for one device's share of a routed MoE feed-forward layer.

This module is shared by the tests, the benchmark and the CPU oracle's callers.  It holds
only input preparation: shapes, seeded normal draws, the fp32 router-logit projection that
produces the layer's input logits, casts to bf16 storage and the symmetric int4 quantiser that
turns fp32 test weights into packed int4 inputs.  It contains none of the layer's own
arithmetic (routing, permutation, expert FFN or combine).

Shapes follow "Systems engineering playbook: optimizing Qwen 3.5-397B MoE on Ironwood (TPU7x)":
hidden size 4096 (section 1, architecture layout), 512 routed experts of intermediate size 1024
with top-10 routing and an always-on shared expert (section 1, sparse MoE), 64 experts per device
under EP=8 (section 3, hybrid sharding), and per-core batches of 64 sequences (decode) or 1024
batched tokens (prefill) over 8 devices (section 2, engine setup).  The int4 format is the
symmetric group-quantised W4A16 format of "vLLM TPU Inference v0.31.0" (4-bit weight scope).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "MoEConfig", "CONFIGS", "make_inputs", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "quantize_int4_sym", "pack_int4", "quantize_fp8_e4m3_channel", "expected_rows_per_group",
    "rows_capacity",
]


@dataclass(frozen=True)
class MoEConfig:
    """One workload: T tokens, hidden H, E global experts, top-k, local experts
    [e_first, e_first + e_local), expert intermediate I."""
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    e_first: int
    e_local: int
    act: str = "bf16"          # "f32" or "bf16": activations and dense weights
    wfmt: str = "dense"        # "dense", "int4" or "fp8" (OCP e4m3, one scale per output channel)
    group_size: int = 128      # int4 quantisation group along K (0: channel-wise, one group of K rows)
    shared_I: int = 0          # intermediate size of the always-on shared expert (0: none)
    zipf_bias: float = 0.0     # additive logit bias zipf_bias * ln(1 / (e + 1)) per expert
    seed: int = 0

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    # Tiny, all experts local, fp32 throughout.
    "tiny": MoEConfig("tiny", T=64, H=256, E=8, k=2, I=128, e_first=0, e_local=8, act="f32"),
    # Decode-shaped EP share: 8 devices x 64 sequences, experts 0-63 of 512 local.
    "decode": MoEConfig("decode", T=512, H=4096, E=512, k=10, I=1024, e_first=0, e_local=64),
    # Prefill-shaped EP share: 8 devices x 1024 batched tokens.
    "prefill": MoEConfig("prefill", T=8192, H=4096, E=512, k=10, I=1024, e_first=0, e_local=64),
    # Zipf-skewed router plus an always-executed shared SwiGLU expert.
    "skewed_shared": MoEConfig("skewed_shared", T=8192, H=4096, E=512, k=10, I=1024, e_first=0,
                               e_local=64, shared_I=1024, zipf_bias=2.0),
    # Prefill shapes with symmetric int4 expert weights, groups of 128 along K, bf16 scales.
    "w4a16": MoEConfig("w4a16", T=8192, H=4096, E=512, k=10, I=1024, e_first=0, e_local=64,
                       wfmt="int4", group_size=128),
    # The int4 format at the decode shape, and channel-wise int4 scales (one group of K rows) at
    # the prefill shape.
    "w4a16_decode": MoEConfig("w4a16_decode", T=512, H=4096, E=512, k=10, I=1024, e_first=0, e_local=64,
                              wfmt="int4", group_size=128),
    "w4a16_channel": MoEConfig("w4a16_channel", T=8192, H=4096, E=512, k=10, I=1024, e_first=0,
                               e_local=64, wfmt="int4", group_size=0),
    # Skewed routing plus the shared expert with int4 routed experts: hot experts of up to 8192
    # rows, where the matrix units bind (the high end of the bf16 / W4A16 comparison).
    "w4a16_skewed": MoEConfig("w4a16_skewed", T=8192, H=4096, E=512, k=10, I=1024, e_first=0, e_local=64,
                              shared_I=1024, zipf_bias=2.0, wfmt="int4", group_size=128),
    # Decode and prefill shapes with FP8 (e4m3) expert weights, one bf16 scale per output channel.
    "fp8_decode": MoEConfig("fp8_decode", T=512, H=4096, E=512, k=10, I=1024, e_first=0, e_local=64,
                            wfmt="fp8"),
    "fp8_prefill": MoEConfig("fp8_prefill", T=8192, H=4096, E=512, k=10, I=1024, e_first=0, e_local=64,
                             wfmt="fp8"),
}


def rows_capacity(cfg: MoEConfig) -> int:
    """Upper bound on the number of local token-expert pairs (each token has k distinct experts)."""
    return cfg.T * min(cfg.k, cfg.e_local)


def expected_rows_per_group(cfg: MoEConfig) -> int:
    """Mean number of pairs per expert under uniform routing (a launch-shape hint only)."""
    return max(1, -(-cfg.T * cfg.k // cfg.E))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 storage bits, round to nearest even (torch's CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 storage bits -> exact fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_int4_sym(w: np.ndarray, group_size: int):
    """Symmetric int4 quantiser for test weights w[K][N] (fp32).

    Per group of `group_size` rows along K and per column n: s = bf16(max|w| / 7) and
    q = clamp(rint(w / s), -8, 7); an all-zero group gets s = 0 and q = 0.
    Returns (q int8 [K][N], scale bits uint16 [K/group_size][N]).
    """
    K, N = w.shape
    assert K % group_size == 0
    g = w.reshape(K // group_size, group_size, N)
    amax = np.abs(g).max(axis=1)                                   # [K/gs][N]
    s_bits = f32_to_bf16_bits((amax / np.float32(7.0)).astype(np.float32))
    s = bf16_bits_to_f32(s_bits)
    safe = np.where(s == 0, np.float32(1.0), s)
    q = np.rint(g / safe[:, None, :]).clip(-8, 7)
    q = np.where(s[:, None, :] == 0, 0, q).astype(np.int8).reshape(K, N)
    return q, s_bits


FP8_E4M3_MAX = 448.0


def quantize_fp8_e4m3_channel(w: np.ndarray):
    """FP8 (OCP e4m3) quantiser for test weights w[K][N] (fp32), one scale per output channel n:
    s = bf16(max_k |w[k][n]| / 448), q = e4m3(clamp(w / s, -448, 448)) rounded to nearest even; an
    all-zero column gets s = 0, q = 0.  Returns (q uint8 [N][K] -- output channel major, each
    column's K bytes contiguous -- and scale bits uint16 [N])."""
    import torch
    amax = np.abs(w).max(axis=0)                                  # [N]
    s_bits = f32_to_bf16_bits((amax / np.float32(FP8_E4M3_MAX)).astype(np.float32))
    s = bf16_bits_to_f32(s_bits)
    safe = np.where(s == 0, np.float32(1.0), s)
    r = np.clip(w / safe[None, :], -FP8_E4M3_MAX, FP8_E4M3_MAX).astype(np.float32)
    r = np.where(s[None, :] == 0, np.float32(0.0), r)
    q = torch.from_numpy(np.ascontiguousarray(r.T)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(q), s_bits


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Pack int4 values q[K][N] (in [-8, 7]) into int32 words [K/8][N]: the two's-complement
    nibble at bits 4i..4i+3 of word [kb][n] holds q[8*kb + i][n]."""
    K, N = q.shape
    assert K % 8 == 0
    nib = (q.astype(np.int32) & 0xF).astype(np.uint32).reshape(K // 8, 8, N)
    word = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        word |= nib[:, i, :] << np.uint32(4 * i)
    return word.view(np.int32)


def _normal(ss: np.random.SeedSequence, shape, scale: float) -> np.ndarray:
    a = np.random.default_rng(ss).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def make_inputs(cfg: MoEConfig, *, tie_quantum: float | None = None,
                rank_perm_seed: int | None = None, threads: int = 8) -> dict:
    """Draw every input of `cfg` from seed `cfg.seed`.

    Draw streams (children of SeedSequence(seed), in this order): x, W_r, then one stream per
    local expert for W_gate, then W_up, then W_down, then the shared expert's gate, up, down.
    All are standard normal fp32 scaled by 1/sqrt(fan_in) (fan_in = H for gate/up/router,
    I for down); x has unit variance.  bf16 configs round x and the dense weights to bf16
    (nearest even).  Router logits are fp32(x) @ W_r in fp32, computed once here, plus the
    optional Zipf bias zipf_bias * ln(1/rank) with rank(e) = e + 1 (or a seeded random rank
    permutation), plus optional rounding to multiples of `tie_quantum` to inject ties.

    Returns a dict of numpy arrays (bf16 tensors are uint16 bit patterns, int4 weights are
    int32 words [e][K/8][N] with uint16 bf16 scales [e][K/gs][N], fp8 weights e4m3 bytes
    [e][N][K] with uint16 bf16 scales [e][N]); the router weight W_r fp32
    [H][E] ("w_router") and, with a Zipf bias, the fp32 bias [E] ("router_bias") come along.
    """
    T, H, E, I, el = cfg.T, cfg.H, cfg.E, cfg.I, cfg.e_local
    ss = np.random.SeedSequence(cfg.seed).spawn(2 + 3 * el + 3)
    s_x, s_r = ss[0], ss[1]
    s_g, s_u, s_d = ss[2:2 + el], ss[2 + el:2 + 2 * el], ss[2 + 2 * el:2 + 3 * el]
    s_sh = ss[2 + 3 * el:]
    bf16 = cfg.act == "bf16"
    assert cfg.act in ("f32", "bf16") and cfg.wfmt in ("dense", "int4", "fp8")
    assert cfg.wfmt == "dense" or bf16, "quantised weights need bf16 activations"

    out: dict = {}
    x = _normal(s_x, (T, H), 1.0)
    if bf16:
        out["x"] = f32_to_bf16_bits(x)
        x = bf16_bits_to_f32(out["x"])
    else:
        out["x"] = x
    wr = _normal(s_r, (H, E), 1.0 / math.sqrt(H))
    out["w_router"] = wr                                          # fp32 [H][E]
    logits = (x @ wr).astype(np.float32)
    if cfg.zipf_bias:
        rank = np.arange(1, E + 1, dtype=np.float64)
        if rank_perm_seed is not None:
            rank = np.random.default_rng(rank_perm_seed).permutation(rank)
        out["router_bias"] = (cfg.zipf_bias * np.log(1.0 / rank)).astype(np.float32)
        logits += out["router_bias"][None, :]
    if tie_quantum:
        logits = (np.rint(logits / np.float32(tie_quantum)) * np.float32(tie_quantum)).astype(np.float32)
    out["logits"] = np.ascontiguousarray(logits, dtype=np.float32)

    def one(args):
        seed, shape, fan_in = args
        w = _normal(seed, shape, 1.0 / math.sqrt(fan_in))
        if cfg.wfmt == "int4":
            q, s_bits = quantize_int4_sym(w, cfg.group_size or shape[0])
            return pack_int4(q), s_bits
        if cfg.wfmt == "fp8":
            return quantize_fp8_e4m3_channel(w)
        return f32_to_bf16_bits(w) if bf16 else w

    jobs = ([(s, (H, I), H) for s in s_g] + [(s, (H, I), H) for s in s_u] +
            [(s, (I, H), I) for s in s_d])
    with ThreadPoolExecutor(max(1, threads)) as ex:
        res = list(ex.map(one, jobs))
    names = ("w_gate", "w_up", "w_down")
    for m, name in enumerate(names):
        part = res[m * el:(m + 1) * el]
        if cfg.wfmt in ("int4", "fp8"):
            out[name] = np.stack([p[0] for p in part])
            out[name + "_scale"] = np.stack([p[1] for p in part])
        else:
            out[name] = np.stack(part)
    if cfg.shared_I:
        Is = cfg.shared_I
        sh = [(s_sh[0], (H, Is), H), (s_sh[1], (H, Is), H), (s_sh[2], (Is, H), Is)]
        for name, (seed, shape, fan_in) in zip(("shared_gate", "shared_up", "shared_down"), sh):
            w = _normal(seed, shape, 1.0 / math.sqrt(fan_in))
            out[name] = f32_to_bf16_bits(w) if bf16 else w
    return out
