"""Benchmark: one device's share of a routed MoE layer on one MI355X.

A step is one pass of the whole path (route -> pack -> permute -> gate/up GEMM + SwiGLU -> down
GEMM [-> shared expert] -> combine) over one batch of synthetic inputs already resident in HBM.
Prints ONE JSON line.  The default workload is the decode-shaped EP share (T=512 tokens, hidden
4096, experts 0-63 of 512 local, top-10, intermediate 1024, bf16).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
  python bench.py --copy-calibration      # plain device copy of known size (HBM counter scale)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed token-expert pairs/s + % of HBM/MFMA roofline, one device's MoE layer"
EVENT_EVERY = 5                                    # timed steps per bracketed gate/up launch
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix peak
FP32_PEAK_TFS = 157.3          # MI355X fp32 vector peak

DESCR = {
    "tiny": "tiny MoE layer, all local: T=64, H=256, 8 experts, top-2, I=128, fp32",
    "decode": "decode-shaped EP share: T=512, H=4096, experts 0-63 of 512 local, top-10, I=1024, bf16",
    "prefill": "prefill-shaped EP share: T=8192, H=4096, experts 0-63 of 512 local, top-10, I=1024, bf16",
    "skewed_shared": "Zipf-skewed routing + shared SwiGLU expert: T=8192, H=4096, 64 of 512 local, "
                     "top-10, I=1024, shared I=1024, bf16",
    "w4a16": "W4A16 prefill EP share: T=8192, H=4096, 64 of 512 local, top-10, I=1024, int4 weights "
             "(group 128, bf16 scales), bf16 activations",
}


def kernel_source_hash() -> str:
    from expert_grouped_gemm_softmax_amd.build import sources
    h = hashlib.sha256()
    for p in sources() + [os.path.join(ROOT, "expert_grouped_gemm_softmax_amd", "csrc", "common.h")]:
        with open(p, "rb") as f:
            h.update(f.read())
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


def gemm_work(cfg, n_loc: int, nonempty: int, op: str):
    """Algorithmic FLOPs and HBM bytes of one grouped-GEMM launch: every weight byte of the
    experts that received pairs read once, activations read once, outputs written once."""
    H, I, T = cfg.H, cfg.I, cfg.T
    act = 2 if cfg.act == "bf16" else 4
    out = 4                                   # expert outputs are written in fp32
    if cfg.wfmt == "int4":
        wbytes = lambda K, N: K * N // 2 + (K // cfg.group_size) * N * 2
    else:
        wbytes = lambda K, N: K * N * act
    if op == "gate_up":
        flops = 4.0 * H * I * n_loc
        byts = nonempty * 2 * wbytes(H, I) + T * H * act + n_loc * I * act
    else:
        flops = 2.0 * H * I * n_loc
        byts = nonempty * wbytes(I, H) + n_loc * I * act + n_loc * H * out
    return flops, byts


def roofline(cfg, flops: float, byts: float, seconds: float):
    peak_f = MFMA_BF16_PEAK_TFS if cfg.act == "bf16" else FP32_PEAK_TFS
    t_hbm = byts / (HBM_PEAK_GBS * 1e9)
    t_mat = flops / (peak_f * 1e12)
    if t_hbm >= t_mat:
        a = byts / seconds / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4)}
    a = flops / seconds / 1e12
    return {"bound": "mfma" if cfg.act == "bf16" else "alu", "achieved": round(a, 1), "peak": peak_f,
            "unit": "TFLOP/s", "frac": round(a / peak_f, 4)}


def cpu_baseline(cfg, inp, budget_s: float):
    """The CPU oracle on a bounded sample of the same workload's tokens (whole path for those
    tokens: routing, blob, permutation, expert FFNs and combine)."""
    import numpy as np
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))

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
            "sample": f"{n} of {cfg.T} tokens drawn uniformly (seed 1), x{reps} repetitions, "
                      f"{pairs} local pairs in {secs:.1f} s on {threads} host threads"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch
    from expert_grouped_gemm_softmax_amd import workloads as W
    from expert_grouped_gemm_softmax_amd.layer import MoELayer, upload

    cfg = W.CONFIGS[args.workload]
    t0 = time.perf_counter()
    inp = W.make_inputs(cfg, threads=16)
    x, logits, wts = upload(inp, cfg, torch.device("cuda:0"))
    layer = MoELayer.from_config(cfg, wts)
    b = layer.buffers(cfg.T, x.device)
    print(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        layer.forward(x, logits)
    torch.cuda.synchronize()
    off = b.group_offsets.cpu().numpy()
    n_loc = int(off[-1])
    nonempty = int((np.diff(off) > 0).sum())

    K = args.steps
    stream = torch.cuda.current_stream()
    # Timed region: K whole steps between synchronisations; HIP events on the launch stream
    # bracket the dominant kernel (the gate/up grouped GEMM) in every EVENT_EVERY-th step, from
    # the first to the last timed step.  A recorded event costs about 3 us of stream time, so
    # bracketing every step would add about 2.5 % to a decode step.
    sampled = list(range(0, K, EVENT_EVERY))
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in sampled}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        e = ev.get(i)
        layer.step_route(logits, b)
        if e:
            e[0].record(stream)
        layer.step_gate_up(x, b)
        if e:
            e[1].record(stream)
        layer.step_down(x, b)
        if cfg.shared_I:
            layer.step_shared(x, b)
        layer.step_combine(b)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per_kernel = {"gate_up": [ev[i][0].elapsed_time(ev[i][1]) * 1e3 for i in sampled]}
    ms_per_step = wall / K * 1e3
    value = n_loc / (ms_per_step / 1e3)

    # Layer latency, measured after the timed region: each step between two events of its own.
    lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        lev[i][0].record(stream)
        layer.forward(x, logits)
        lev[i][1].record(stream)
    torch.cuda.synchronize()
    step_us = np.array([lev[i][0].elapsed_time(lev[i][1]) * 1e3 for i in range(K)])

    # Per-step breakdown, measured after the timed region (events between every step).
    names = ["route_pack_permute", "gate_up", "down"] + (["shared"] if cfg.shared_I else []) + ["combine"]
    steps = [lambda: layer.step_route(logits, b), lambda: layer.step_gate_up(x, b),
             lambda: layer.step_down(x, b)] + ([lambda: layer.step_shared(x, b)] if cfg.shared_I else []) + \
            [lambda: layer.step_combine(b)]
    nb = max(3, min(K, 10))
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(nb)]
    for i in range(nb):
        bev[i][0].record(stream)
        for j, fn in enumerate(steps):
            fn()
            bev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    breakdown = {n: float(np.mean([bev[i][j].elapsed_time(bev[i][j + 1]) * 1e3 for i in range(nb)]))
                 for j, n in enumerate(names)}

    gu_us = float(np.mean(per_kernel["gate_up"]))
    flops, byts = gemm_work(cfg, n_loc, nonempty, "gate_up")
    roof = roofline(cfg, flops, byts, gu_us * 1e-6)
    roof["kernel"] = "grouped GEMM gate/up + SwiGLU"
    roof["algorithmic_bytes"] = int(byts)
    roof["algorithmic_flops"] = int(flops)
    roof["traffic"] = measured_traffic(args.workload, "gate_up")
    dn_us = breakdown["down"]
    dflops, dbytes = gemm_work(cfg, n_loc, nonempty, "down")
    layer_flops = flops + dflops
    layer_bytes = byts + dbytes

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "pairs/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic: seeded normal activations, random-init expert weights, fp32 router logits",
        "config": {"workload": DESCR[args.workload], "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
                   "I": cfg.I, "e_local": cfg.e_local, "weights": cfg.wfmt, "shared_I": cfg.shared_I},
        "roofline": roof,
        "roofline_samples": len(sampled),
        "n_local_pairs": n_loc,
        "latency_us": {"median": round(float(np.median(step_us)), 1),
                       "p10": round(float(np.percentile(step_us, 10)), 1),
                       "p90": round(float(np.percentile(step_us, 90)), 1)},
        "kernels_us": {n: round(v, 1) for n, v in breakdown.items()},
        "down_roofline": roofline(cfg, dflops, dbytes, dn_us * 1e-6),
        "gemm_pair_roofline": roofline(cfg, layer_flops, layer_bytes, (gu_us + dn_us) * 1e-6),
    }
    att = attainable_peaks()
    out["attainable"] = att
    if att:
        if roof["unit"] == "GB/s":
            roof["frac_of_attainable"] = round(roof["achieved"] / att["hbm_read_gbs"], 4)
        elif roof["bound"] == "mfma":
            roof["frac_of_attainable"] = round(roof["achieved"] / att["mfma_bf16_tflops"], 4)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
