"""Benchmark: one device's share of a routed MoE layer on one MI355X.

A step is one pass of the whole path (route -> pack -> permute -> gate/up GEMM + SwiGLU -> down
GEMM [-> shared expert] -> combine) over one batch of synthetic inputs already resident in HBM.
Prints ONE JSON line.  The headline workload is the largest one that fits one GPU: Zipf-skewed
routing plus a shared SwiGLU expert (T=8192 tokens, hidden 4096, experts 0-63 of 512 local, top-10,
intermediate 1024, bf16).  The other four workloads (tiny fp32, decode, prefill, W4A16) are
measured the same way, each in a child process of its own that runs before this process touches
the GPU (so a profiler's per-process kernel statistics of this process cover the headline only),
and reported under "workloads".

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--cpu-seconds S]
  python bench.py --workload NAME          # one workload only, as the headline
  python bench.py --copy-calibration       # plain device copy of known size (HBM counter scale)
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed token-expert pairs/s + % of HBM/MFMA roofline, one device's MoE layer"
HEADLINE = "skewed_shared"
SUBS = ["tiny", "decode", "prefill", "w4a16", "w4a16_decode", "w4a16_channel", "w4a16_skewed", "fp8_decode",
        "fp8_prefill"]
EVENT_EVERY = 5                # timed steps per event-bracketed launch of the dominant kernel
# Warm-up runs the requested steps and, if they take less, more until this much time has passed:
# after the idle seconds of input generation the first ~15 steps of a workload run up to 8 %
# slower while the GPU's clocks come back up (kernel traces), and the timed region should see
# the steady state.
MIN_WARMUP_S = 0.25
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_16BIT_PEAK_TFS = 2500.0   # MI355X dense bf16 / fp16 matrix peak
FP32_PEAK_TFS = 157.3          # MI355X fp32 vector peak

DESCR = {
    "tiny": "tiny MoE layer, all local: T=64, H=256, 8 experts, top-2, I=128, fp32",
    "decode": "decode-shaped EP share: T=512, H=4096, experts 0-63 of 512 local, top-10, I=1024, bf16",
    "prefill": "prefill-shaped EP share: T=8192, H=4096, experts 0-63 of 512 local, top-10, I=1024, bf16",
    "skewed_shared": "Zipf-skewed routing + shared SwiGLU expert: T=8192, H=4096, 64 of 512 local, "
                     "top-10, I=1024, shared I=1024, bf16",
    "w4a16": "W4A16 prefill EP share: T=8192, H=4096, 64 of 512 local, top-10, I=1024, int4 weights "
             "(group 128, bf16 scales), bf16 activations",
    "w4a16_decode": "decode-shaped EP share with int4 expert weights (group 128, bf16 scales): T=512, "
                    "H=4096, 64 of 512 local, top-10, I=1024, bf16 activations",
    "w4a16_channel": "prefill-shaped EP share with channel-wise int4 expert weights (one bf16 scale per "
                     "output column): T=8192, H=4096, 64 of 512 local, top-10, I=1024, bf16 activations",
    "w4a16_skewed": "Zipf-skewed routing + shared SwiGLU expert with int4 routed experts (group 128): "
                    "T=8192, H=4096, 64 of 512 local, top-10, I=1024, shared I=1024 (bf16)",
    "fp8_decode": "decode-shaped EP share with FP8 (e4m3) expert weights, one bf16 scale per output "
                  "channel: T=512, H=4096, 64 of 512 local, top-10, I=1024, bf16 activations",
    "fp8_prefill": "prefill-shaped EP share with FP8 (e4m3) expert weights, one bf16 scale per output "
                   "channel: T=8192, H=4096, 64 of 512 local, top-10, I=1024, bf16 activations",
}


def kernel_source_hash() -> str:
    """Hash of the library's sources with comments and whitespace removed: counter profiles taken on
    other code are not reported, edits of comments alone do not invalidate them."""
    from expert_grouped_gemm_softmax_amd.build import sources
    h = hashlib.sha256()
    for p in sources() + [os.path.join(ROOT, "expert_grouped_gemm_softmax_amd", "csrc", "common.h")]:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)      # block comments
        text = re.sub(r"//[^\n]*", " ", text)                    # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when absent or taken on
    different kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel_src") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------------------------
# Algorithmic work
# ---------------------------------------------------------------------------------------------
def weight_bytes(cfg, K: int, N: int) -> int:
    """Bytes of one K x N expert matrix as stored in HBM (int4 words + bf16 scales, or dense)."""
    if cfg.wfmt == "int4":
        return K * N // 2 + (K // (cfg.group_size or K)) * N * 2
    if cfg.wfmt == "fp8":
        return K * N + N * 2
    return K * N * (2 if cfg.act == "bf16" else 4)


def work(cfg, n_loc: int, nonempty: int) -> dict:
    """Algorithmic flops and bytes: the layer (weights of the experts that received pairs, the
    shared expert's weights, x read once, the router logits, y written once in fp32) and each
    kernel (its weights and its reads of x; the implementation's own h and o round trips are
    not algorithmic)."""
    H, I, T, E, Is = cfg.H, cfg.I, cfg.T, cfg.E, cfg.shared_I
    act = 2 if cfg.act == "bf16" else 4
    x_b, logit_b, y_b = T * H * act, T * E * 4, T * H * 4
    gu_w = nonempty * 2 * weight_bytes(cfg, H, I)
    dn_w = nonempty * weight_bytes(cfg, I, H)
    sh_w = 3 * H * Is * act
    w = {
        "gate_up": {"flops": 4.0 * H * I * n_loc, "bytes": gu_w + x_b},
        "down": {"flops": 2.0 * H * I * n_loc, "bytes": dn_w},
        "layer": {"flops": 6.0 * H * I * n_loc + 6.0 * H * Is * T,
                  "bytes": gu_w + dn_w + sh_w + x_b + logit_b + y_b},
    }
    if Is:
        w["shared"] = {"flops": 6.0 * H * Is * T, "bytes": sh_w + x_b}
    return w


def matrix_peak(cfg) -> float:
    return MFMA_16BIT_PEAK_TFS if cfg.act == "bf16" else FP32_PEAK_TFS


def roofline(cfg, flops: float, byts: float, seconds: float, att=None) -> dict:
    """Achieved rate against the binding roofline (HBM if bytes/BW >= flops/peak, else the matrix
    peak of the arithmetic dtype; fp32 arithmetic runs on the vector ALU) for work done in
    `seconds`; frac_of_attainable against the measured ceilings when given."""
    peak_f = matrix_peak(cfg)
    t_hbm = byts / (HBM_PEAK_GBS * 1e9)
    t_mat = flops / (peak_f * 1e12)
    if t_hbm >= t_mat:
        a = byts / seconds / 1e9
        r = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(a / HBM_PEAK_GBS, 4)}
        if att:
            r["frac_of_attainable"] = round(a / att["hbm_read_gbs"], 4)
    else:
        a = flops / seconds / 1e12
        r = {"bound": "mfma" if cfg.act == "bf16" else "alu", "achieved": round(a, 1), "peak": peak_f,
             "unit": "TFLOP/s", "frac": round(a / peak_f, 4)}
        if att and cfg.act == "bf16":
            r["frac_of_attainable"] = round(a / att["mfma_bf16_tflops"], 4)
    return r


def layer_roofline(cfg, wk: dict, seconds: float) -> dict:
    """max(B/BW, F/P) / t for the whole layer: the fraction of the layer's own roofline time."""
    L = wk["layer"]
    t_hbm = L["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mat = L["flops"] / (matrix_peak(cfg) * 1e12)
    return {"bytes": int(L["bytes"]), "flops": int(L["flops"]), "t_hbm_us": round(t_hbm * 1e6, 1),
            "t_matrix_us": round(t_mat * 1e6, 1), "bound": "hbm" if t_hbm >= t_mat else
            ("mfma" if cfg.act == "bf16" else "alu"), "frac": round(max(t_hbm, t_mat) / seconds, 4)}


# ---------------------------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores
# ---------------------------------------------------------------------------------------------
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_threads() -> int:
    """Every core this process may use: its CPU affinity, capped by a cgroup CPU quota when one is
    set, and by os.cpu_count()."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, -(-int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    return max(1, min(n, os.cpu_count() or n))


def cpu_baseline(cfg, inp, budget_s: float):
    """The CPU oracle on a bounded sample of the same workload's tokens (the whole path for those
    tokens: routing, blob, permutation, expert FFNs and combine), one thread per usable core."""
    import numpy as np
    import oracle
    threads = host_threads()

    def run(tokens):
        t0 = time.perf_counter()
        ids, w = oracle.route(inp["logits"][tokens], cfg.k)
        blob = oracle.pack(ids, w)
        sp, off, pp = oracle.permute(blob, cfg.e_first, cfg.e_local)
        sub = dict(inp, x=inp["x"][tokens])
        oracle.layer(sub, cfg.with_(T=len(tokens)), ids, w, threads=threads)
        return time.perf_counter() - t0, int(off[-1])

    rng = np.random.default_rng(1)
    probe = np.sort(rng.choice(cfg.T, size=min(cfg.T, 2 * threads), replace=False))
    t_probe, _ = run(probe)
    n = int(min(cfg.T, max(len(probe), len(probe) * budget_s / max(t_probe, 1e-6))))
    tokens = np.sort(rng.choice(cfg.T, size=n, replace=False))
    secs, pairs, reps = 0.0, 0, 0
    while reps == 0 or secs < budget_s:                    # repeat small workloads to fill the budget
        dt, n_pairs = run(tokens)
        secs, pairs, reps = secs + dt, pairs + n_pairs, reps + 1
    return {"value": round(pairs / secs, 2), "unit": "pairs/s", "cores": threads, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"{n} of {cfg.T} tokens drawn uniformly (seed 1), x{reps} repetitions, "
                      f"{pairs} local pairs in {secs:.1f} s on {threads} host threads"}


# ---------------------------------------------------------------------------------------------
# Measured ceilings
# ---------------------------------------------------------------------------------------------
def attainable_peaks():
    """Measured ceilings on this GPU, next to the published peaks: a bf16 MFMA loop that touches no
    memory and a streaming read of 2 GiB (well past the 256 MB last-level cache), each the best
    of a few launches.  None if the calibration library is not built."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "expert_grouped_gemm_softmax_amd", "libmoe_calib.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.moe_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.moe_calib_mfma_flops.restype = ctypes.c_double
    lib.moe_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")

    def best(launch, reps=5):
        launch()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    blocks, iters = cus * 4, 20000
    t = best(lambda: lib.moe_calib_mfma(blocks, iters, ctypes.c_void_p(sink.data_ptr()), sp))
    mfma = lib.moe_calib_mfma_flops(blocks, iters) / t / 1e12
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gbs = 0.0
    for wg_per_cu in (2, 4, 8):
        blk = cus * wg_per_cu
        if nbytes % (blk * 256 * 8 * 16):
            continue
        t = best(lambda: lib.moe_calib_read(ctypes.c_void_p(buf.data_ptr()), nbytes, blk,
                                            ctypes.c_void_p(sink.data_ptr()), sp))
        gbs = max(gbs, nbytes / t / 1e9)
    del buf
    torch.cuda.synchronize()
    return {"hbm_read_gbs": round(gbs, 1), "mfma_bf16_tflops": round(mfma, 1),
            "how": "best of 5 launches: 2 GiB streaming read (16-byte nontemporal loads, 8 in flight per "
                   "lane); bf16 16x16x32 MFMA loop on registers, 8 independent accumulators per wave"}


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 5}))


# ---------------------------------------------------------------------------------------------
# One workload
# ---------------------------------------------------------------------------------------------
def measure(name: str, steps: int, warmup: int, cpu_s: float | None, att=None, min_warmup_s: float = MIN_WARMUP_S) -> dict:
    """Time `steps` whole steps of one workload (after `warmup`), then per-step latencies and a
    per-kernel breakdown in separate event-bracketed passes; rooflines; the CPU oracle."""
    import numpy as np
    import torch
    from expert_grouped_gemm_softmax_amd import workloads as W
    from expert_grouped_gemm_softmax_amd.layer import MoELayer, upload

    cfg = W.CONFIGS[name]
    t0 = time.perf_counter()
    inp = W.make_inputs(cfg, threads=16)
    x, logits, wts = upload(inp, cfg, torch.device("cuda:0"))
    layer = MoELayer.from_config(cfg, wts)
    b = layer.buffers(cfg.T, x.device)
    print(f"[bench] {name}: inputs ready in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)

    for _ in range(warmup):
        layer.forward(x, logits)
    torch.cuda.synchronize()
    warm_run, t_warm = warmup, time.perf_counter()
    while time.perf_counter() - t_warm < min_warmup_s:
        for _ in range(5):
            layer.forward(x, logits)
        torch.cuda.synchronize()
        warm_run += 5
    off = b.group_offsets.cpu().numpy()
    n_loc = int(off[-1])
    nonempty = int((np.diff(off) > 0).sum())

    K = steps
    stream = torch.cuda.current_stream()
    # Timed region: K whole steps between synchronisations; HIP events on the launch stream
    # bracket the dominant kernel (the routed gate/up grouped GEMM) in every EVENT_EVERY-th step,
    # from the first to the last timed step (a recorded event costs about 3 us of stream time).
    sampled = list(range(0, K, EVENT_EVERY))
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in sampled}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        e = ev.get(i)
        layer.step_route(logits, b, stream)
        if e:
            e[0].record(stream)
        layer.step_gate_up(x, b, stream)
        if e:
            e[1].record(stream)
        layer.step_down(x, b, stream)
        if cfg.shared_I:
            layer.step_shared(x, b, stream)
        layer.step_combine(b, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gu_us = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) * 1e3 for i in sampled]))
    ms_per_step = wall / K * 1e3

    # Layer latency, after the timed region: each step between two events of its own.
    lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        lev[i][0].record(stream)
        layer.forward(x, logits)
        lev[i][1].record(stream)
    torch.cuda.synchronize()
    step_us = np.array([lev[i][0].elapsed_time(lev[i][1]) * 1e3 for i in range(K)])

    # Per-kernel breakdown, after the timed region (events between every step).
    names = ["route_pack_permute", "gate_up", "down"] + (["shared"] if cfg.shared_I else []) + ["combine"]
    fns = [lambda: layer.step_route(logits, b, stream), lambda: layer.step_gate_up(x, b, stream),
           lambda: layer.step_down(x, b, stream)] + \
          ([lambda: layer.step_shared(x, b, stream)] if cfg.shared_I else []) + \
          [lambda: layer.step_combine(b, stream)]
    nb = max(3, min(K, 10))
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(nb)]
    for i in range(nb):
        bev[i][0].record(stream)
        for j, fn in enumerate(fns):
            fn()
            bev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    kus = {n: float(np.mean([bev[i][j].elapsed_time(bev[i][j + 1]) * 1e3 for i in range(nb)]))
           for j, n in enumerate(names)}

    # The two GEMMs launched back to back, 10 launches between two events: per-launch kernel time
    # without an event's dispatch wait in front of each launch (which inflates a bracketed
    # 100-us kernel by several percent; the kernel traces agree with these figures).
    b2b = {}
    for n, fn in (("gate_up", lambda: layer.step_gate_up(x, b, stream)),
                  ("down", lambda: layer.step_down(x, b, stream))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        b2b[n] = e0.elapsed_time(e1) * 1e3 / 10

    # The router projection x W_r (+ bias) and routing from the hidden states (moe_route_hidden),
    # timed apart from the step: the workloads' own steps start from the router logits.
    from expert_grouped_gemm_softmax_amd import ops
    wsplit = ops.prepare_router_weights(torch.from_numpy(inp["w_router"]).to(x.device))
    rbias = torch.from_numpy(inp["router_bias"]).to(x.device) if "router_bias" in inp else None
    r_logits = torch.empty_like(logits)
    for _ in range(3):
        ops.route_hidden(x, wsplit, cfg.k, bias=rbias, logits=r_logits, blob=b.blob, write_ids=False)
    rev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nb)]
    for i in range(nb):
        rev[i][0].record(stream)
        ops.router_logits(x, wsplit, bias=rbias, logits=r_logits)
        rev[i][1].record(stream)
        ops.route_packed(r_logits, cfg.k, blob=b.blob, write_ids=False)
        rev[i][2].record(stream)
    torch.cuda.synchronize()
    proj_us = float(np.mean([rev[i][0].elapsed_time(rev[i][1]) * 1e3 for i in range(nb)]))
    topk_us = float(np.mean([rev[i][1].elapsed_time(rev[i][2]) * 1e3 for i in range(nb)]))
    del wsplit, r_logits

    # The same step with the dense weights left in their stated [e][K][N] layout (transposed
    # operand reads, bf16 h) beside the prepared layout's
    stated = None
    if cfg.wfmt == "dense" and cfg.act == "bf16" and not cfg.shared_I:
        xs, ls, kn = upload(inp, cfg, x.device, stated_layout=True)
        lk = MoELayer.from_config(cfg, kn)
        for _ in range(3):
            lk.forward(xs, ls)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            lk.forward(xs, ls)
        torch.cuda.synchronize()
        stated = round((time.perf_counter() - t0) / K * 1e3, 4)
        del lk, kn, xs, ls

    wk = work(cfg, n_loc, nonempty)
    roof = roofline(cfg, wk["gate_up"]["flops"], wk["gate_up"]["bytes"], gu_us * 1e-6, att)
    b2b_roof = roofline(cfg, wk["gate_up"]["flops"], wk["gate_up"]["bytes"], b2b["gate_up"] * 1e-6, att)
    roof.update({"kernel": "routed grouped GEMM gate/up + SwiGLU", "time_us": round(gu_us, 1),
                 "algorithmic_bytes": int(wk["gate_up"]["bytes"]), "algorithmic_flops": int(wk["gate_up"]["flops"]),
                 "traffic": measured_traffic(name, "gate_up"), "samples": len(sampled),
                 "back_to_back": {"time_us": round(b2b["gate_up"], 1), "achieved": b2b_roof["achieved"],
                                  "frac": b2b_roof["frac"]}})
    kernels = {"down": roofline(cfg, wk["down"]["flops"], wk["down"]["bytes"], b2b["down"] * 1e-6, att)}
    kernels["down"]["time_us"] = round(b2b["down"], 1)
    if cfg.shared_I:
        kernels["shared"] = roofline(cfg, wk["shared"]["flops"], wk["shared"]["bytes"], kus["shared"] * 1e-6, att)
    pair_s = n_loc / (ms_per_step / 1e3)
    res = {
        "workload": name, "description": DESCR[name],
        "config": {"T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I, "e_local": cfg.e_local,
                   "weights": cfg.wfmt, "act": cfg.act, "shared_I": cfg.shared_I},
        "ms_per_step": round(ms_per_step, 4), "pairs_per_s": round(pair_s, 1), "steps": K, "warmup": warmup, "warmup_steps_run": warm_run,
        "timed_region_s": round(wall, 4), "n_local_pairs": n_loc, "nonempty_experts": nonempty,
        "latency_us": {"p10": round(float(np.percentile(step_us, 10)), 1),
                       "median": round(float(np.median(step_us)), 1),
                       "p90": round(float(np.percentile(step_us, 90)), 1)},
        "layer_roofline": layer_roofline(cfg, wk, ms_per_step * 1e-3),
        "roofline": roof,
        "kernels_us": {n: round(v, 1) for n, v in kus.items()},
        "kernel_rooflines": kernels,
        "stated_layout_ms_per_step": stated,
        "router_from_hidden": {
            "projection_us": round(proj_us, 1), "route_packed_us": round(topk_us, 1),
            "projection_roofline": roofline(cfg, 2.0 * cfg.T * cfg.H * cfg.E,
                                            cfg.T * cfg.H * (2 if cfg.act == "bf16" else 4) + cfg.H * cfg.E * 4
                                            + cfg.T * cfg.E * 4, proj_us * 1e-6, att),
            "note": "x W_r (+ bias) with W_r as two bf16 planes (2 MFMA products per weight), then "
                    "top-k routing; not part of the step, which starts from the router logits"},
    }
    if cpu_s:
        print(f"[bench] {name}: timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, inp, cpu_s)
    else:
        res["cpu_baseline"] = None
    del layer, b, x, logits, wts
    torch.cuda.empty_cache()
    return res


def run_child(name: str, args) -> dict:
    """One sub-workload in a child process of its own (this process has not touched the GPU)."""
    cmd = [sys.executable, "-u", os.path.abspath(__file__), "--child", "--workload", name,
           "--steps", str(args.steps), "--warmup", str(args.warmup), "--cpu-seconds", str(args.cpu_seconds),
           "--min-warmup-s", str(args.min_warmup_s)]
    if args.no_cpu_baseline:
        cmd.append("--no-cpu-baseline")
    print(f"[bench] child: {name}", file=sys.stderr, flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"bench child for {name} failed with exit code {r.returncode}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="measure this workload only (as the headline)")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--min-warmup-s", type=float, default=MIN_WARMUP_S,
                    help="warm-up continues past --warmup steps until this many seconds have passed "
                         "(0 for counter runs, which need few dispatches)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    cpu_s = None if args.no_cpu_baseline else args.cpu_seconds
    if args.child:
        print(json.dumps(measure(args.workload, args.steps, args.warmup, cpu_s, min_warmup_s=args.min_warmup_s)), flush=True)
        return

    print(f"[bench] pid {os.getpid()}", file=sys.stderr, flush=True)
    head = args.workload or HEADLINE
    subs = {} if args.workload else {n: run_child(n, args) for n in SUBS}   # before this process uses the GPU

    att = attainable_peaks()
    h = measure(head, args.steps, args.warmup, None if cpu_s is None else max(cpu_s, 12.0), att,
                min_warmup_s=args.min_warmup_s)
    for r in subs.values():                       # measured ceilings of this machine for the children too
        if att:
            for rr in [r["roofline"]] + list(r["kernel_rooflines"].values()):
                if rr["unit"] == "GB/s":
                    rr["frac_of_attainable"] = round(rr["achieved"] / att["hbm_read_gbs"], 4)
                elif rr["bound"] == "mfma":
                    rr["frac_of_attainable"] = round(rr["achieved"] / att["mfma_bf16_tflops"], 4)
    out = {
        "metric": METRIC, "value": h["pairs_per_s"], "unit": "pairs/s", "n_gpus": 1, "steps": h["steps"],
        "warmup": h["warmup"], "warmup_steps_run": h["warmup_steps_run"], "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if h["config"]["act"] == "bf16" else "f32",
        "data": "synthetic: seeded normal activations, random-init expert weights, fp32 router logits",
        "config": {"workload": f"{head}: {DESCR[head]}", **h["config"]},
        "roofline": h["roofline"],
        "cpu_baseline": h["cpu_baseline"],
        "layer_roofline": h["layer_roofline"],
        "latency_us": h["latency_us"],
        "kernels_us": h["kernels_us"],
        "kernel_rooflines": h["kernel_rooflines"],
        "n_local_pairs": h["n_local_pairs"],
        "timed_region_s": h["timed_region_s"],
        "attainable": att,
        "workloads": {head: {k: v for k, v in h.items() if k not in ("workload",)}, **subs},
    }
    # bf16 vs W4A16 expert weights on the same routing (the weight-format rule's measurements)
    wl = out["workloads"]
    out["format_rule"] = {
        f"{a}/{b}": {"rows_per_expert": round(wl[a]["n_local_pairs"] / wl[a]["config"]["e_local"], 1),
                     "bf16_ms": wl[a]["ms_per_step"], "w4a16_ms": wl[b]["ms_per_step"],
                     "bf16_over_w4a16": round(wl[a]["ms_per_step"] / wl[b]["ms_per_step"], 3)}
        for a, b in (("decode", "w4a16_decode"), ("prefill", "w4a16"), ("skewed_shared", "w4a16_skewed"))
        if a in wl and b in wl}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
