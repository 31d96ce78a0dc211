"""Benchmark: dropless MoE layer forward on one MI355X.

Workload: the Mixtral-8x7B-shaped layer (T=4096 tokens, H=4096, E=8 experts, top-2 softmax
router in fp32, SwiGLU F=14336, bf16 activations and weights), synthetic seeded inputs resident
in HBM.  One step = one full layer forward through the library's fused entry point
(route -> permute -> grouped SwiGLU GEMMs -> combine).

Prints ONE JSON line: tokens/s over the timed steps, active TFLOP/s, per-stage times from HIP
events recorded by the library on the compute stream, the roofline of the dominant kernel (the
first grouped GEMM with the fused SwiGLU epilogue), and the CPU oracle timed on a bounded sample.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd active TFLOPS + tokens/s at 1 GPU; % of MFMA / HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
STAGES = ["route", "permute", "gemm1_swiglu", "gemm2", "shared_expert", "combine"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm1_swiglu_mixtral_8x7b_hbm_traffic.txt")
GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_layer_fp32_amd", "csrc", "gemm.hip")


def measured_traffic():
    """HBM bytes per launch of the first grouped GEMM from the committed PMC summary, or None
    when the kernel source changed since the counters were taken."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if kv.get("gemm_source_sha256") != sha or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def _hip():
    h = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def algorithmic(cfg):
    """Useful FLOPs and the bytes each stage must move at the ABI boundary (bf16 = 2 B)."""
    T, H, E, k, F, Fs = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    R = T * k
    a = 2  # bf16 bytes
    return {
        "route": dict(flops=2 * T * H * E, bytes=T * H * a + H * E * 4 + R * 8),
        "permute": dict(flops=0, bytes=T * H * a + R * 4 + R * H * a + R * 8 + (E + 1) * 4),
        "gemm1_swiglu": dict(flops=4 * R * H * F, bytes=R * H * a + E * H * 2 * F * a + R * F * a),
        "gemm2": dict(flops=2 * R * F * H, bytes=R * F * a + E * F * H * a + R * H * a),
        "shared_expert": dict(flops=6 * T * H * Fs, bytes=(T * H * a * 2 + 3 * H * Fs * a) if Fs else 0),
        "combine": dict(flops=0, bytes=R * H * a + R * 8 + T * H * a),
        "active_flops": 2 * T * H * E + 6 * R * H * F + 6 * T * H * Fs,
    }


def cpu_baseline(cfg, d, sample_tokens):
    """The float64 oracle (as it stands) on the first `sample_tokens` tokens of the same layer."""
    import numpy as np
    from oracle import moe
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    x = d["x"][:sample_tokens].float().cpu().numpy()
    wr = d["w_router"].cpu().numpy()
    w1 = [d["w1"][e].float().cpu().numpy() for e in range(cfg.E)]
    w2 = [d["w2"][e].float().cpu().numpy() for e in range(cfg.E)]
    t0 = time.perf_counter()
    moe.forward(x, wr, lambda e: w1[e], lambda e: w2[e], E=cfg.E, k=cfg.k, score=cfg.score, norm=cfg.norm)
    dt = time.perf_counter() - t0
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of the same layer (all {cfg.E} experts' weights widened "
                      f"to float64 inside the oracle); {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-sample-tokens", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (for scaling HBM counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": 1 << 30, "launches": args.steps}))
        return
    import moe_inputs
    import mixture_experts_layer_fp32_amd as moe_gpu
    from mixture_experts_layer_fp32_amd import _lib

    cfg = moe_inputs.CONFIGS["mixtral_8x7b"]
    dev = "cuda"
    d = moe_inputs.make_inputs(cfg, seed=0, weight_device=dev, act_device=dev)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    x = d["x"]
    c_layer = layer.c_struct(x.dtype)
    L = _lib.lib()
    need = L.moe_workspace_size(ctypes.byref(c_layer), cfg.T)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    hip = _hip()
    K, W = args.steps, args.warmup
    events = []
    for _ in range(K):
        row = []
        for _ in range(7):
            ev = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(ev)) == 0
            row.append(ev)
        events.append(row)

    def step(ev_row=None):
        dbg = None
        if ev_row is not None:
            dbg = _lib.MoeDebugC()
            for i, ev in enumerate(ev_row):
                dbg.stage_events[i] = ev.value
        st = L.moe_forward(ctypes.byref(c_layer), ctypes.c_void_p(x.data_ptr()), cfg.T,
                           ctypes.c_void_p(y.data_ptr()), ctypes.byref(dbg) if dbg is not None else None,
                           ctypes.c_void_p(ws.data_ptr()), need, ctypes.c_void_p(stream.cuda_stream))
        _lib.check("moe_forward", st)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    stage_ms = {s: [] for s in STAGES}
    for row in events:
        for i, s in enumerate(STAGES):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), row[i], row[i + 1]) == 0
            stage_ms[s].append(ms.value)
    for row in events:
        for ev in row:
            hip.hipEventDestroy(ev)
    avg_ms = {s: sum(v) / len(v) for s, v in stage_ms.items()}
    alg = algorithmic(cfg)
    ms_per_step = elapsed * 1e3 / K
    tokens_per_s = cfg.T * K / elapsed
    active_tflops = alg["active_flops"] / (ms_per_step * 1e-3) / 1e12

    stages = {}
    for s in STAGES:
        ms = avg_ms[s]
        if ms <= 0 or (alg[s]["flops"] == 0 and alg[s]["bytes"] == 0):
            continue
        rec = {"us": round(ms * 1e3, 2), "GB_s": round(alg[s]["bytes"] / (ms * 1e-3) / 1e9, 1)}
        if alg[s]["flops"]:
            rec["TFLOP_s"] = round(alg[s]["flops"] / (ms * 1e-3) / 1e12, 1)
        if s.startswith("gemm"):
            rec["frac_mfma_peak"] = round(rec["TFLOP_s"] / PEAK_BF16_TFLOPS, 4)
        else:
            rec["frac_hbm_peak"] = round(rec["GB_s"] / PEAK_HBM_GBS, 4)
        stages[s] = rec
    g1 = alg["gemm1_swiglu"]
    g1_tflops = g1["flops"] / (avg_ms["gemm1_swiglu"] * 1e-3) / 1e12
    roofline = {"kernel": "gemm_bf16_kernel<256,swiglu> (grouped GEMM1 + fused SwiGLU)", "bound": "mfma",
                "achieved": round(g1_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g1_tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                "flops_per_launch": g1["flops"], "avg_launch_us": round(avg_ms["gemm1_swiglu"] * 1e3, 2)}
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.description, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "F": cfg.F,
                   "router": "fp32 softmax top-2", "parallelism": "single GPU"},
        "active_tflops": round(active_tflops, 1),
        "frac_bf16_mfma_peak": round(active_tflops / PEAK_BF16_TFLOPS, 4),
        "stages": stages,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
