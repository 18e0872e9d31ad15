"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bit-exact: top-k ids, routing weights, the routing blob, sorted_pairs[:n_loc], group_offsets and
pair_pos (given identical fp32 logits).  Layer output: relative L2 <= 1e-2 and
max |y - y_oracle| <= 3e-2 * RMS(y_oracle).  Mid-size shapes and the five full workload shapes
are checked on every token, the full shapes with both tile families; the largest accepted
activation matrix on sampled tokens plus properties that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
from expert_grouped_gemm_softmax_amd import ops
from expert_grouped_gemm_softmax_amd import workloads as W
from expert_grouped_gemm_softmax_amd.layer import MoELayer, upload

pytestmark = pytest.mark.gpu

REL_L2, MAX_ABS_RMS = 1e-2, 3e-2


def _dev():
    return torch.device("cuda:0")


def _np(t):
    return t.cpu().numpy()


def _check_routing(b, inp, cfg):
    ids, w = oracle.route(inp["logits"], cfg.k)
    blob = oracle.pack(ids, w)
    sp, off, pp = oracle.permute(blob, cfg.e_first, cfg.e_local)
    assert np.array_equal(_np(b.ids), ids), "top-k ids"
    assert np.array_equal(_np(b.w).view(np.int32), w.view(np.int32)), "routing weight bits"
    assert np.array_equal(_np(b.blob), blob), "routing blob"
    assert np.array_equal(_np(b.group_offsets), off), "group offsets"
    assert np.array_equal(_np(b.sorted_pairs)[:len(sp)], sp), "sorted pairs"
    assert np.array_equal(_np(b.pair_pos), pp), "pair positions"
    return ids, w, off


def _check_close(got, ref, what=""):
    rms = float(np.sqrt((ref ** 2).mean()))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(got - ref).max())
    print(f"{what}: rel_l2={rel:.3e} max_abs/rms={mx / max(rms, 1e-300):.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert rel <= REL_L2, rel
    assert mx <= MAX_ABS_RMS * rms, mx / rms


def _run(cfg, inp, y_dtype=torch.float32, m_hint=None, h_dtype=torch.float16):
    x, logits, wts = upload(inp, cfg, _dev(), h_dtype=h_dtype)
    layer = MoELayer.from_config(cfg, wts, y_dtype=y_dtype)
    if m_hint is not None:
        layer.m_hint = lambda T: m_hint
    y = layer.forward(x, logits)
    torch.cuda.synchronize()
    return layer, layer.buffers(cfg.T, x.device), y


# ----------------------------------------------------------------------------------------------
# Routing, blob and permutation: bit-exact
# ----------------------------------------------------------------------------------------------
def _route_only(cfg, logits_np):
    logits = torch.from_numpy(logits_np).to(_dev())
    ids, w = ops.route(logits, cfg.k)
    blob = ops.pack_routing(ids, w)
    sp, off, pp = ops.permute(blob, cfg.e_first, cfg.e_local)
    torch.cuda.synchronize()
    r_ids, r_w = oracle.route(logits_np, cfg.k)
    r_blob = oracle.pack(r_ids, r_w)
    r_sp, r_off, r_pp = oracle.permute(r_blob, cfg.e_first, cfg.e_local)
    assert np.array_equal(_np(ids), r_ids)
    assert np.array_equal(_np(w).view(np.int32), r_w.view(np.int32))
    assert np.array_equal(_np(blob), r_blob)
    assert np.array_equal(_np(off), r_off)
    assert np.array_equal(_np(sp)[:len(r_sp)], r_sp)
    assert np.array_equal(_np(pp), r_pp)
    return r_off


def _logits_only(cfg, tie_quantum=None, rank_perm_seed=None):
    # router logits only (no expert weights are drawn): same recipe as workloads.make_inputs
    c = cfg.with_(e_local=1, I=64, shared_I=0, wfmt="dense")
    return W.make_inputs(c, tie_quantum=tie_quantum, rank_perm_seed=rank_perm_seed)["logits"]


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_routing_bit_exact_on_every_workload(name):
    cfg = W.CONFIGS[name]
    off = _route_only(cfg, _logits_only(cfg))
    print(name, "n_loc", off[-1], "empty groups", int((np.diff(off) == 0).sum()))


@pytest.mark.parametrize("name,tq", [("decode", 0.25), ("prefill", 0.5), ("tiny", 0.25)])
def test_routing_bit_exact_with_injected_ties(name, tq):
    cfg = W.CONFIGS[name]
    _route_only(cfg, _logits_only(cfg, tie_quantum=tq))


def test_routing_bit_exact_random_rank_zipf():
    cfg = W.CONFIGS["skewed_shared"]
    _route_only(cfg, _logits_only(cfg, rank_perm_seed=1))


@pytest.mark.parametrize("T,E,k,e_first,e_local", [
    (1, 4, 1, 0, 4), (3, 7, 7, 2, 5), (77, 64, 1, 0, 64), (129, 1024, 64, 0, 1024),
    (1000, 1024, 10, 512, 512), (257, 513, 33, 100, 413), (4096, 96, 6, 0, 1),
    (65536, 512, 10, 64, 64), (5000, 128, 8, 120, 8), (64, 8, 2, 0, 8),
    (2048, 64, 8, 0, 64), (2049, 64, 8, 8, 40), (3000, 1024, 16, 0, 1024)])
def test_routing_bit_exact_edge_shapes(T, E, k, e_first, e_local):
    rng = np.random.default_rng(T + E + k)
    L = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    L[: max(1, T // 7)] = np.rint(L[: max(1, T // 7)])          # heavy ties in some rows
    if T > 2:
        L[1, :] = -0.0
        L[2, ::3] = 0.0
    cfg = W.MoEConfig("edge", T=T, H=64, E=E, k=k, I=64, e_first=e_first, e_local=e_local)
    _route_only(cfg, L)


@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (333, 96, 7), (4096, 512, 10), (1, 1024, 64)])
def test_route_packed_equals_route_then_pack(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    L = torch.from_numpy((rng.standard_normal((T, E)) * 2).astype(np.float32)).to(_dev())
    ids, w = ops.route(L, k)
    blob = ops.pack_routing(ids, w)
    ids2, w2, blob2 = ops.route_packed(L, k)
    _, _, blob3 = ops.route_packed(L, k, write_ids=False)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(blob, blob2) and torch.equal(blob, blob3)


@pytest.mark.parametrize("E,K,N,dt", [(1, 64, 64, torch.bfloat16), (3, 4096, 1024, torch.bfloat16),
                                       (2, 1024, 4096, torch.bfloat16), (5, 100, 37, torch.float32),
                                       (1, 1, 1, torch.float32)])
def test_prepare_dense_weights_is_a_transpose(E, K, N, dt):
    g = torch.Generator().manual_seed(E * K + N)
    w = torch.randn((E, K, N), generator=g).to(dt).to(_dev())
    out = ops.prepare_dense_weights(w)
    torch.cuda.synchronize()
    ref = w.transpose(1, 2).contiguous()
    assert out.shape == (E, N, K) and torch.equal(out.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                                                   ref.view(torch.int16 if dt == torch.bfloat16 else torch.int32))


def test_fp32_gemm_reads_both_dense_layouts_identically():
    cfg = MID["f32"]
    inp = W.make_inputs(cfg)
    x, logits, wts = upload(inp, cfg, _dev())
    layer = MoELayer.from_config(cfg, wts)
    layer.forward(x, logits)
    b = layer.buffers(cfg.T, _dev())
    wg, wu = (torch.from_numpy(inp[n]).to(_dev()) for n in ("w_gate", "w_up"))      # stated [E][K][N]
    h2 = torch.empty_like(b.h)
    ops.grouped_gemm(0, x, b.group_offsets, wg, wu, h2, K=cfg.H, N=cfg.I, row_index=b.sorted_pairs,
                     row_div=cfg.k, weights_nk=False)
    torch.cuda.synchronize()
    n = int(b.group_offsets[-1])
    assert torch.equal(h2[:n].view(torch.int32), b.h[:n].view(torch.int32))


def _permute_vs_oracle(ids, e_first, e_local):
    T, k = ids.shape
    blob_np = oracle.pack(ids.astype(np.int32), np.full((T, k), 1.0 / k, np.float32))
    sp, off, pp = ops.permute(torch.from_numpy(blob_np).to(_dev()), e_first, e_local)
    torch.cuda.synchronize()
    r_sp, r_off, r_pp = oracle.permute(blob_np, e_first, e_local)
    assert np.array_equal(_np(off), r_off)
    assert np.array_equal(_np(sp)[:len(r_sp)], r_sp)
    assert np.array_equal(_np(pp), r_pp)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 511, 512, 1500, 2047, 2048])
def test_permute_distinct_experts_token_counts(T):
    # every token routes to k distinct experts (as top-k does); token counts around 32-token words
    rng = np.random.default_rng(T)
    k, E = 8, 200
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    for e_first, e_local in [(0, 64), (37, 64), (150, 50), (0, 1), (10, 65)]:
        _permute_vs_oracle(ids, e_first, e_local)


@pytest.mark.parametrize("T,k", [(300, 6), (2000, 8), (5, 64), (3000, 6)])
def test_permute_repeated_experts_within_a_token(T, k):
    # the permutation is defined for any ids, including a token that names one expert twice
    rng = np.random.default_rng(T * k)
    ids = rng.integers(0, 40, size=(T, k))
    ids[0, :] = 7                                               # one token, all slots one expert
    for e_first, e_local in [(4, 24), (0, 40), (0, 100)]:
        _permute_vs_oracle(ids, e_first, e_local)


def test_permute_with_no_local_pair():
    T, k = 50, 4
    ids = np.stack([np.arange(100, 104)] * T).astype(np.int32)
    blob = torch.from_numpy(oracle.pack(ids, np.full((T, k), 0.25, np.float32))).to(_dev())
    sp = torch.full((T * k,), -7, dtype=torch.int32, device=_dev())
    sp, off, pp = ops.permute(blob, 0, 16, sorted_pairs=sp)
    torch.cuda.synchronize()
    assert np.all(_np(off) == 0) and np.all(_np(pp) == -1) and np.all(_np(sp) == -7)


# ----------------------------------------------------------------------------------------------
# Full layer, mid-size shapes: every token
# ----------------------------------------------------------------------------------------------
MID = {
    "bf16_ragged": W.MoEConfig("mid", T=300, H=512, E=64, k=6, I=384, e_first=8, e_local=24),
    "bf16_all_local_k1": W.MoEConfig("mid", T=333, H=256, E=16, k=1, I=192, e_first=0, e_local=16),
    "bf16_skew_empty": W.MoEConfig("mid", T=257, H=384, E=48, k=4, I=256, e_first=0, e_local=16,
                                   zipf_bias=3.0),
    "bf16_shared": W.MoEConfig("mid", T=200, H=512, E=32, k=4, I=128, e_first=4, e_local=12,
                               shared_I=320),
    "int4_g128": W.MoEConfig("mid", T=280, H=512, E=32, k=4, I=256, e_first=0, e_local=16,
                             wfmt="int4", group_size=128),
    "int4_channel": W.MoEConfig("mid", T=150, H=256, E=16, k=3, I=256, e_first=2, e_local=8,
                                    wfmt="int4", group_size=256),
    # groups narrower than a 64-k chunk: several scale rows per chunk, one per word row
    "int4_g32": W.MoEConfig("mid", T=220, H=512, E=24, k=4, I=256, e_first=0, e_local=12,
                            wfmt="int4", group_size=32),
    "int4_g8": W.MoEConfig("mid", T=90, H=256, E=8, k=2, I=128, e_first=0, e_local=8,
                           wfmt="int4", group_size=8),
    # decode-shaped tiles with about 40 rows per expert: two 32-row tiles per expert, so the down
    # projection has four tiles per workgroup and its loads run across three tile boundaries
    "bf16_many_tiles_per_workgroup": W.MoEConfig("mid", T=320, H=4096, E=64, k=8, I=256, e_first=0,
                                                 e_local=64),
    # more than 64 local experts: the prefill down tiles fall back to the LDS tile table
    "bf16_80_local_experts": W.MoEConfig("mid", T=160, H=512, E=128, k=8, I=128, e_first=16, e_local=80),
    # the most local experts the library accepts: tile tables of 1024 groups (the prefill down
    # projection falls back to the LDS tile table)
    "bf16_1024_local_experts": W.MoEConfig("mid", T=600, H=256, E=1024, k=8, I=128, e_first=0, e_local=1024),
    # fp8 (e4m3) weights with per-column scales, converted exactly to the 16-bit operand type
    "fp8": W.MoEConfig("mid", T=260, H=512, E=32, k=4, I=384, e_first=0, e_local=16, wfmt="fp8"),
    "fp8_many_tiles": W.MoEConfig("mid", T=300, H=1024, E=64, k=8, I=256, e_first=8, e_local=40, wfmt="fp8"),
    "f32": W.MoEConfig("mid", T=130, H=256, E=12, k=3, I=192, e_first=1, e_local=9, act="f32"),
    "f32_shared": W.MoEConfig("mid", T=70, H=128, E=8, k=2, I=64, e_first=0, e_local=8, act="f32",
                              shared_I=128),
}


MID_BF16_H = [n for n, c in MID.items() if c.act == "bf16" and c.wfmt in ("dense", "fp8")]


@pytest.mark.parametrize("variant", ["small_m", "large_m"])
@pytest.mark.parametrize("name,h", [(n, "f16") for n in MID] + [(n, "bf16") for n in MID_BF16_H])
def test_layer_mid_size_every_token(name, h, variant):
    """Every token of the mid-size shapes on both tile families; bf16 layers with fp16 h (the
    default) and, over bf16 down weights, with bf16 h."""
    cfg = MID[name]
    inp = W.make_inputs(cfg)
    h_dtype = torch.float16 if h == "f16" else torch.bfloat16
    layer, b, y = _run(cfg, inp, y_dtype=torch.float32, m_hint=(8 if variant == "small_m" else 0), h_dtype=h_dtype)
    if cfg.act == "bf16":
        assert b.h.dtype == h_dtype
    ids, w, off = _check_routing(b, inp, cfg)
    ref = oracle.layer(inp, cfg, ids, w, threads=8)
    _check_close(_np(y).astype(np.float64), ref, f"{name}/{h}/{variant}")
    if not cfg.shared_I:
        counts = np.zeros(cfg.T, int)
        loc = (ids >= cfg.e_first) & (ids < cfg.e_first + cfg.e_local)
        counts = loc.sum(1)
        assert np.all(_np(y)[counts == 0] == 0.0)


def test_layer_on_two_side_streams_matches_the_default_stream():
    # every kernel goes on the caller's stream, and calls on different streams (separate buffers)
    # may run at the same time: both results equal the default-stream result bit for bit
    cfg = MID["bf16_ragged"]
    inp = W.make_inputs(cfg)
    x, logits, wts = upload(inp, cfg, _dev())
    y0 = MoELayer.from_config(cfg, wts).forward(x, logits).clone()
    torch.cuda.synchronize()
    layers = [MoELayer.from_config(cfg, wts) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]          # default priority
    outs = []
    for layer, s in zip(layers, streams):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            outs.append(layer.forward(x, logits, stream=s))
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(y.view(torch.int32), y0.view(torch.int32))


def test_layer_bf16_output_is_rounded_fp32_output_and_deterministic():
    """The bf16 layer output is the round-to-nearest-even of the fp32 output (the combine
    accumulates in fp32 either way), and repeated calls are bitwise identical."""
    cfg = MID["bf16_ragged"]
    inp = W.make_inputs(cfg)
    x, logits, wts = upload(inp, cfg, _dev())
    l32 = MoELayer.from_config(cfg, wts, y_dtype=torch.float32)
    l16 = MoELayer.from_config(cfg, wts, y_dtype=torch.bfloat16)
    y32a = l32.forward(x, logits).clone()
    y16a = l16.forward(x, logits).clone()
    y32b = l32.forward(x, logits).clone()
    y16b = l16.forward(x, logits).clone()
    torch.cuda.synchronize()
    assert torch.equal(y32a.view(torch.int32), y32b.view(torch.int32))
    assert torch.equal(y16a.view(torch.int16), y16b.view(torch.int16))
    assert torch.equal(y16a.view(torch.int16), y32a.to(torch.bfloat16).view(torch.int16))
    ids, w = oracle.route(inp["logits"], cfg.k)
    ref = oracle.layer(inp, cfg, ids, w, threads=8)
    _check_close(y32a.cpu().numpy().astype(np.float64), ref, "fp32 out")


@pytest.mark.parametrize("hint", [8, 1 << 20], ids=["decode_tiles", "prefill_tiles"])
@pytest.mark.parametrize("name,h_dtype", [("bf16_ragged", torch.float16), ("bf16_ragged", torch.bfloat16),
                                          ("bf16_skew_empty", torch.float16), ("bf16_shared", torch.float16),
                                          ("bf16_shared", torch.bfloat16), ("int4_g128", torch.float16)])
def test_down_projection_16bit_output_and_16bit_combine(name, h_dtype, hint):
    """DOWN with 16-bit output rows (h's dtype) is the round-to-nearest-even of its fp32 output
    (same accumulators, only the epilogue's store differs), on both tile families; combine on
    those rows (and 16-bit shared rows) matches the oracle within the layer bar."""
    cfg = MID[name]
    inp = W.make_inputs(cfg)
    x, logits, wts = upload(inp, cfg, _dev(), h_dtype=h_dtype)
    layer = MoELayer.from_config(cfg, wts)
    layer.m_hint = lambda T: hint
    layer.forward(x, logits)
    b = layer.buffers(cfg.T, x.device)
    assert b.h.dtype == h_dtype
    Wt = layer.weights
    def down(out_dtype, shared=False):
        if shared:
            out = torch.empty(b.shared_o.shape, dtype=out_dtype, device=x.device)
            return ops.grouped_gemm(1, b.shared_h, b.shared_offsets, Wt.shared_down, None, out, K=cfg.shared_I,
                                    N=cfg.H, m_hint=cfg.T)
        out = torch.empty(b.o.shape, dtype=out_dtype, device=x.device)
        return ops.grouped_gemm(1, b.h, b.group_offsets, Wt.w_down, None, out, K=cfg.I, N=cfg.H, s0=Wt.s_down,
                                group_size=Wt.group_size, m_hint=hint)

    o16, o32 = down(h_dtype), down(torch.float32)
    sh16 = sh32 = None
    if cfg.shared_I:
        sh16, sh32 = down(h_dtype, shared=True), down(torch.float32, shared=True)
    y = ops.combine(o16, b.blob, b.pair_pos, sh16, y_dtype=torch.float32)
    torch.cuda.synchronize()
    n = int(b.group_offsets[-1])
    bits = torch.int16
    assert torch.equal(o16[:n].view(bits), o32[:n].to(h_dtype).view(bits))
    if sh16 is not None:
        assert torch.equal(sh16.view(bits), sh32.to(h_dtype).view(bits))
    ids, w = oracle.route(inp["logits"], cfg.k)
    ref = oracle.layer(inp, cfg, ids, w, threads=8)
    _check_close(_np(y).astype(np.float64), ref, f"{name} h {h_dtype} 16-bit o")


@pytest.mark.parametrize("hint", [8, 1 << 20], ids=["decode_tiles", "prefill_tiles"])
@pytest.mark.parametrize("name", ["bf16_ragged", "bf16_skew_empty", "bf16_all_local_k1",
                                  "bf16_many_tiles_per_workgroup", "bf16_80_local_experts"])
def test_stated_layout_weights_equal_the_prepared_layout(name, hint):
    """Dense bf16 weights in the stated [e][K][N] layout (MOE_W_DENSE, transposed operand reads)
    give the same bits as the prepared [e][N][K] copy (the same products in the same order) for
    gate/up with bf16 and fp16 h and for the down projection over bf16 h, on both tile families;
    the layer on them matches the oracle."""
    cfg = MID[name]
    inp = W.make_inputs(cfg)
    x, logits, kn = upload(inp, cfg, _dev(), stated_layout=True)
    _, _, nk = upload(inp, cfg, _dev(), h_dtype=torch.bfloat16)
    layer = MoELayer.from_config(cfg, kn)
    layer.m_hint = lambda T: hint
    y = layer.forward(x, logits)
    b = layer.buffers(cfg.T, x.device)
    assert b.h.dtype == torch.bfloat16
    n = b.group_offsets[-1]
    for h_dtype in (torch.bfloat16, torch.float16):
        h1 = torch.empty(b.h.shape, dtype=h_dtype, device=x.device)
        h2 = torch.empty_like(h1)
        ops.grouped_gemm(0, x, b.group_offsets, kn.w_gate, kn.w_up, h1, K=cfg.H, N=cfg.I, row_index=b.sorted_pairs,
                         row_div=cfg.k, m_hint=hint, weights_nk=False)
        ops.grouped_gemm(0, x, b.group_offsets, nk.w_gate, nk.w_up, h2, K=cfg.H, N=cfg.I, row_index=b.sorted_pairs,
                         row_div=cfg.k, m_hint=hint)
        torch.cuda.synchronize()
        assert torch.equal(h1[:n].view(torch.int16), h2[:n].view(torch.int16))
    o1 = torch.empty((b.h.shape[0], cfg.H), dtype=torch.float32, device=x.device)
    o2 = torch.empty_like(o1)
    ops.grouped_gemm(1, b.h, b.group_offsets, kn.w_down, None, o1, K=cfg.I, N=cfg.H, m_hint=hint, weights_nk=False)
    ops.grouped_gemm(1, b.h, b.group_offsets, nk.w_down, None, o2, K=cfg.I, N=cfg.H, m_hint=hint)
    torch.cuda.synchronize()
    assert torch.equal(o1[:n].view(torch.int32), o2[:n].view(torch.int32))
    ids, w = oracle.route(inp["logits"], cfg.k)
    _check_close(_np(y).astype(np.float64), oracle.layer(inp, cfg, ids, w, threads=8), f"{name} stated layout")


def test_stated_layout_full_decode_every_token():
    """The decode workload with its weights in the stated [e][K][N] layout, every token."""
    cfg = W.CONFIGS["decode"]
    inp = W.make_inputs(cfg, threads=16)
    x, logits, kn = upload(inp, cfg, _dev(), stated_layout=True)
    layer = MoELayer.from_config(cfg, kn)
    y = layer.forward(x, logits)
    torch.cuda.synchronize()
    ids, w, off = _check_routing(layer.buffers(cfg.T, x.device), inp, cfg)
    _check_close(_np(y).astype(np.float64), oracle.layer(inp, cfg, ids, w, threads=ORACLE_THREADS),
                 "decode stated layout all 512 tokens")


# More than 16,384 pairs: the multi-kernel permutation with its caller workspace.
GRAPH_LARGE_PERMUTE = W.MoEConfig("mid", T=2100, H=256, E=64, k=8, I=128, e_first=0, e_local=32)


@pytest.mark.parametrize("variant", ["small_m", "large_m"])
@pytest.mark.parametrize("name", ["bf16_ragged", "bf16_shared", "int4_g128", "fp8", "large_permute"])
def test_layer_step_replays_from_a_captured_graph(name, variant):
    """The library launches kernels only (no allocation, memset or synchronisation), so a whole
    layer step captured in a graph replays bit for bit like the eager step.  Each replay follows
    eager work that clears the step's buffers and runs another layer, and is checked."""
    cfg = GRAPH_LARGE_PERMUTE if name == "large_permute" else MID[name]
    print(f"graph capture: {name} {variant} T={cfg.T} pairs={cfg.T * cfg.k}", flush=True)
    inp = W.make_inputs(cfg)
    x, logits, wts = upload(inp, cfg, _dev())
    layer = MoELayer.from_config(cfg, wts)
    other = MoELayer.from_config(cfg, wts)
    if variant == "small_m":
        layer.m_hint = lambda T: 8
    y_eager = layer.forward(x, logits).clone()      # the eager step also allocates the buffers
    torch.cuda.synchronize()
    b = layer.buffers(cfg.T, x.device)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_graph = layer.forward(x, logits)
    torch.cuda.synchronize()
    for rep in range(3):
        for buf in (b.y, b.o, b.h, b.sorted_pairs, b.pair_pos, b.group_offsets, b.blob):
            buf.zero_()
        other.forward(x * (rep + 2), logits)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int32), y_eager.view(torch.int32)), f"replay {rep}"


def test_layer_single_token_and_single_expert():
    cfg = W.MoEConfig("one", T=1, H=128, E=4, k=2, I=64, e_first=1, e_local=1)
    inp = W.make_inputs(cfg)
    layer, b, y = _run(cfg, inp, y_dtype=torch.float32)
    ids, w, off = _check_routing(b, inp, cfg)
    ref = oracle.layer(inp, cfg, ids, w)
    if off[-1] == 0:
        assert np.all(_np(y) == 0)
    else:
        _check_close(_np(y).astype(np.float64), ref, "T=1")


# ----------------------------------------------------------------------------------------------
# Full workload shapes: every token, both tile families (the decode-shaped 32-row tiles and the
# prefill-shaped 256-row tiles), against one oracle evaluation
# ----------------------------------------------------------------------------------------------
ORACLE_THREADS = 16


def _sample_tokens(cfg, ids, n=40):
    loc = ((ids >= cfg.e_first) & (ids < cfg.e_first + cfg.e_local)).sum(1)
    T = cfg.T
    pick = set(range(6)) | set(range(T - 6, T)) | set(np.linspace(0, T - 1, n - 16).astype(int).tolist())
    pick |= {int(np.argmax(loc)), int(np.argmin(loc))}
    return np.array(sorted(pick), np.int32), loc


def _both_families(cfg, inp):
    """The layer with the tile family its shape selects and with the other one forced; routing is
    checked bit for bit on both.  Returns (ids, w, offsets, {family: y as float64 numpy})."""
    x, logits, wts = upload(inp, cfg, _dev())
    out = {}
    for fam, hint in (("decode_tiles", 8), ("prefill_tiles", 1 << 20)):
        layer = MoELayer.from_config(cfg, wts, y_dtype=torch.float32)
        layer.m_hint = lambda T, h=hint: h
        y = layer.forward(x, logits)
        torch.cuda.synchronize()
        b = layer.buffers(cfg.T, x.device)
        ids, w, off = _check_routing(b, inp, cfg)
        out[fam] = _np(y).astype(np.float64)
        del layer, b, y
    del x, logits, wts
    torch.cuda.empty_cache()
    return ids, w, off, out


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "w4a16", "w4a16_decode", "w4a16_channel",
                                  "fp8_decode", "fp8_prefill"])
def test_layer_full_workload_every_token(name):
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg, threads=16)
    ids, w, off, ys = _both_families(cfg, inp)
    ref = oracle.layer(inp, cfg, ids, w, threads=ORACLE_THREADS)
    loc = ((ids >= cfg.e_first) & (ids < cfg.e_first + cfg.e_local)).sum(1)
    for fam, yn in ys.items():
        _check_close(yn, ref, f"{name}/{fam} all {cfg.T} tokens")
        assert np.all(yn[loc == 0] == 0.0)
    print(name, "n_loc", int(off[-1]), "empty groups", int((np.diff(off) == 0).sum()),
          "max group", int(np.diff(off).max()))


SKEW_PARTS = 4


@pytest.fixture(scope="module")
def skewed_run():
    cfg = W.CONFIGS["skewed_shared"]
    inp = W.make_inputs(cfg, threads=16)
    ids, w, off, ys = _both_families(cfg, inp)
    return cfg, inp, ids, w, off, ys


@pytest.mark.parametrize("part", range(SKEW_PARTS))
def test_layer_skewed_shared_every_token(skewed_run, part):
    """The skewed workload (hot experts of up to 8192 rows, so the grouped-M tile order with more
    than four m-tiles per expert runs; empty experts; the shared expert on every token): every
    token, in four contiguous quarters, both tile families."""
    cfg, inp, ids, w, off, ys = skewed_run
    toks = np.arange(part * cfg.T // SKEW_PARTS, (part + 1) * cfg.T // SKEW_PARTS, dtype=np.int32)
    ref = oracle.layer(inp, cfg, ids, w, tokens=toks, threads=ORACLE_THREADS)
    for fam, yn in ys.items():
        _check_close(yn[toks], ref, f"skewed_shared/{fam} tokens {toks[0]}..{toks[-1]}")
    if part == 0:
        sizes = np.diff(off)
        print("skewed_shared n_loc", int(off[-1]), "empty groups", int((sizes == 0).sum()),
              "max group", int(sizes.max()), "experts with > 4 m-tiles of 256 rows", int((sizes > 1024).sum()))
        assert (sizes > 4 * 256).sum() >= 1        # the grouped-M order past its first group runs


def test_layer_int4_skewed_shared_first_quarter():
    """int4 routed experts under the skewed routing (hot experts of up to 8192 rows on the
    192-row int4 tiles, empty experts) plus the dense shared expert: the first 2048 tokens on
    both tile families."""
    cfg = W.CONFIGS["w4a16_skewed"]
    inp = W.make_inputs(cfg, threads=16)
    ids, w, off, ys = _both_families(cfg, inp)
    toks = np.arange(cfg.T // 4, dtype=np.int32)
    ref = oracle.layer(inp, cfg, ids, w, tokens=toks, threads=ORACLE_THREADS)
    for fam, yn in ys.items():
        _check_close(yn[toks], ref, f"w4a16_skewed/{fam} tokens 0..{toks[-1]}")
    assert np.all(np.isfinite(ys["prefill_tiles"]))


# ----------------------------------------------------------------------------------------------
# The largest activation matrix the library accepts: the down projection's input h (written by
# the gate/up GEMM) just under 2^31 bytes, so its last rows sit at the top of the kernels' 32-bit
# byte offsets (both tile families)
# ----------------------------------------------------------------------------------------------
MAX_ROWS = W.MoEConfig("max_rows", T=(1 << 31) // (8192 * 2) - 1, H=256, E=8, k=1, I=8192, e_first=0,
                       e_local=8)


@pytest.fixture(scope="module")
def max_rows_inputs():
    return W.make_inputs(MAX_ROWS, threads=16)


@pytest.mark.parametrize("variant", ["small_m", "large_m"])
def test_layer_at_the_largest_activation_matrix(max_rows_inputs, variant):
    cfg, inp = MAX_ROWS, max_rows_inputs
    layer, b, y = _run(cfg, inp, m_hint=(8 if variant == "small_m" else 0))
    ids, w, off = _check_routing(b, inp, cfg)
    n_loc = int(off[-1])
    assert n_loc == cfg.T and n_loc * cfg.I * 2 < (1 << 31) <= (n_loc + 1) * cfg.I * 2
    toks, loc = _sample_tokens(cfg, ids)
    last = int(_np(b.sorted_pairs)[n_loc - 1])         # the pair whose h row is the last one
    toks = np.unique(np.concatenate([toks, [last // cfg.k]])).astype(np.int32)
    ref = oracle.layer(inp, cfg, ids, w, tokens=toks, threads=8)
    yn = y[torch.from_numpy(toks).long().to(y.device)].float().cpu().numpy().astype(np.float64)
    _check_close(yn, ref, f"max_rows/{variant}")
    del layer, b, y
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------------------------
# Router projection on the GPU (logits = x W_r (+ bias)) before routing
# ----------------------------------------------------------------------------------------------
def _router_case(cfg):
    c = cfg.with_(e_local=1, I=64, shared_I=0, wfmt="dense")     # router inputs only
    inp = W.make_inputs(c)
    x = _upload_x(inp, cfg)
    wr = torch.from_numpy(inp["w_router"]).to(_dev())
    bias = torch.from_numpy(inp["router_bias"]).to(_dev()) if "router_bias" in inp else None
    return inp, x, wr, bias


def _upload_x(inp, cfg):
    if cfg.act == "bf16":
        return torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16).to(_dev())
    return torch.from_numpy(inp["x"]).to(_dev())


@pytest.mark.parametrize("T,H,E", [(100, 512, 128), (100, 320, 128), (37, 4096, 64), (1, 256, 64)])
def test_router_logits_small_batches(T, H, E):
    """The projection's small-batch tiles (16 rows with four chunks in registers when H is a
    multiple of 256, else 32 rows with two), every logit within the bound moe.h states."""
    cfg = W.MoEConfig("router", T=T, H=H, E=E, k=2, I=64, e_first=0, e_local=1)
    inp, x, wr, bias = _router_case(cfg)
    logits = ops.router_logits(x, ops.prepare_router_weights(wr), bias=bias)
    torch.cuda.synchronize()
    ref = oracle.router_logits(inp["x"], inp["w_router"], inp.get("router_bias"))
    xf = W.bf16_bits_to_f32(inp["x"])
    absum = np.abs(xf.astype(np.float64)) @ np.abs(inp["w_router"].astype(np.float64))
    bound = (2.0 ** -18 + (H // 32 + 32 + 2) * 2.0 ** -24) * absum + 2 * np.spacing(np.abs(ref).astype(np.float32))
    err = np.abs(_np(logits).astype(np.float64) - ref)
    print(f"router T={T} H={H} E={E}: max err/bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_router_projection_and_routing_from_hidden_states(name):
    """moe_route_hidden on every workload: each logit within the derived error bound of the
    oracle's fp64 projection, routing on the GPU's logits bit-exact against the oracle routing the
    same logits, top-k ids equal to the oracle's wherever the bound decides them, and weights
    within the error budget that follows from the logits' bound."""
    cfg = W.CONFIGS[name]
    inp, x, wr, bias = _router_case(cfg)
    wsplit = ops.prepare_router_weights(wr)
    logits, ids, w, blob = ops.route_hidden(x, wsplit, cfg.k, bias=bias)
    torch.cuda.synchronize()
    g_logits, g_ids, g_w = _np(logits), _np(ids), _np(w)
    # the projection against the oracle, element by element
    ref = oracle.router_logits(inp["x"], inp["w_router"], inp.get("router_bias"))
    xf = W.bf16_bits_to_f32(inp["x"]) if cfg.act == "bf16" else inp["x"]
    absum = np.abs(xf.astype(np.float64)) @ np.abs(inp["w_router"].astype(np.float64))
    # the bound moe.h states: rounding steps of the fp32 sums (MFMA path: one per 32-product step
    # and up to 32 inside a step, plus the sum of the two planes; fp32 path: one per product)
    mfma = cfg.act == "bf16" and cfg.H % 64 == 0 and cfg.E % 64 == 0
    n_acc = (cfg.H // 32 + 32 + 2) if mfma else (cfg.H + 2)
    bound = (2.0 ** -18 + n_acc * 2.0 ** -24) * absum + 2 * np.spacing(np.abs(ref).astype(np.float32))
    err = np.abs(g_logits.astype(np.float64) - ref)
    print(f"{name}: max |logit err| {err.max():.3e}, max err/bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)
    # routing of the GPU's own logits: bit-exact (the logits-in path)
    r_ids, r_w = oracle.route(g_logits, cfg.k)
    assert np.array_equal(g_ids, r_ids) and np.array_equal(g_w.view(np.int32), r_w.view(np.int32))
    assert np.array_equal(_np(blob), oracle.pack(r_ids, r_w))
    # against the oracle's own logits: ids where decidable, weights within the budget
    o_ids, o_w = oracle.route(ref, cfg.k)
    T, k = o_ids.shape
    srt = -np.sort(-ref.astype(np.float64), axis=1)
    bmax = bound.max(axis=1)
    gap_ok = (srt[:, k - 1] - srt[:, k] > 2 * bmax) if cfg.E > k else np.ones(T, bool)
    same_set = np.array([set(a) == set(b) for a, b in zip(g_ids, o_ids)])
    assert np.all(same_set[gap_ok])
    order_ok = gap_ok & np.all(srt[:, :k - 1] - srt[:, 1:k] > 2 * bmax[:, None], axis=1)
    assert np.array_equal(g_ids[order_ok], o_ids[order_ok])
    budget = 4 * bmax[:, None] * o_w + 8 * np.spacing(o_w)
    assert np.all(np.abs(g_w[order_ok].astype(np.float64) - o_w[order_ok]) <= budget[order_ok])
    print(f"{name}: decided sets {gap_ok.mean():.4f}, decided order {order_ok.mean():.4f}, "
          f"sets equal overall {same_set.mean():.4f}")
