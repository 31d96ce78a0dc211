"""Benchmark: dropless MoE layer forward on one MI355X.

Default workload: the Mixtral-8x7B-shaped layer (T=4096 tokens, H=4096, E=8 experts, top-2
softmax router in fp32, SwiGLU F=14336, bf16 activations and weights), synthetic seeded inputs
resident in HBM.  One step = one full layer forward through the library's fused entry point
(route -> permute -> grouped SwiGLU GEMMs -> shared expert -> combine).  ``--workload`` selects
another of the layer shapes (Qwen3-235B, DeepSeek-V3 in bf16 or with e4m3 experts, the tiny fp32
layer) for the same measurement.

Prints ONE JSON line: tokens/s over the timed steps, active TFLOP/s, per-stage times from HIP
events recorded by the library on the compute stream, the roofline of the dominant kernel (the
first grouped GEMM with the fused SwiGLU epilogue), and the CPU oracle timed on a bounded sample.

With --backward a step is one call of the layer backward instead (gradients of x and of every
weight for a dy drawn from its own seed, routing state from one untimed forward); the line then
carries the backward's stages and the roofline of its longest expert GEMM.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--backward] [--no-cpu-baseline]
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
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0, "fp8": 5000.0}  # MI355X dense MFMA by operand type
PEAK_BF16_TFLOPS = PEAK_TFLOPS["bf16"]
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
STAGES = ["route", "permute", "gemm1_swiglu", "gemm2", "shared_expert", "combine"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm1_swiglu_mixtral_8x7b_hbm_traffic.txt")
# the first grouped GEMM's kernel is built from these files
GEMM_SOURCES = [os.path.join(ROOT, "mixture_experts_layer_fp32_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_common.hpp", "common.hpp")]


def gemm_source_sha256():
    """SHA-256 of the GEMM sources with // comments and blank lines removed (a comment edit does
    not change the kernel the counters were taken on)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        for line in open(f, encoding="utf-8"):
            code = re.sub(r"//.*", "", line).strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "wgrad_w1_backward_mixtral_8x7b_hbm_traffic.txt")
BWD_SOURCES = [os.path.join(ROOT, "mixture_experts_layer_fp32_amd", "csrc", f)
               for f in ("backward.hip", "gemm_common.hpp", "common.hpp")]


def backward_source_sha256():
    """SHA-256 of the backward GEMM's sources, // comments and blank lines removed."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in BWD_SOURCES:
        for line in open(f, encoding="utf-8"):
            code = re.sub(r"//.*", "", line).strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_backward_traffic():
    """HBM bytes per launch of the backward's dW1 GEMM from the committed PMC summary, or None
    when its sources changed since the counters were taken."""
    if not os.path.exists(BWD_TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(BWD_TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.get("backward_source_sha256") != backward_source_sha256() or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def measured_traffic():
    """HBM bytes per launch of the first grouped GEMM from the committed PMC summary, or None
    when the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.get("gemm_source_sha256") != gemm_source_sha256() or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def _hip():
    h = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def algorithmic(cfg, active_experts=None):
    """Useful FLOPs and the bytes each stage of the fused forward must move (unique HBM bytes).

    Activations in the config's dtype (bf16 2 B, fp32 4 B); weights and the permuted / hidden
    rows of the e4m3 path 1 B plus one fp32 scale per 128 values (weights: per 128 x 128 block).
    Only experts that received rows are streamed (``active_experts``, default all E).
    """
    T, H, E, k, F, Fs = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    R = T * k
    Ea = E if active_experts is None else active_experts
    fp8 = cfg.w_dtype == "fp8"
    a = 4 if cfg.act_dtype == "f32" else 2
    rowb = (lambda n: n + n // 128 * 4) if fp8 else (lambda n: n * a)   # one row of n values
    wbytes = (lambda K, N: K * N + (K // 128) * (N // 128) * 4) if fp8 else (lambda K, N: K * N * a)
    sh = bool(Fs)
    return {
        "route": dict(flops=2 * T * H * E, bytes=T * H * a + H * E * 4 + R * 8 + (E * 4 if cfg.zipf_bias else 0)),
        # the fused forward writes no permuted copy: dispatch = ids -> maps (+ the e4m3 path's
        # per-token quantisation of x), and GEMM1 gathers the token rows it needs
        "permute": dict(flops=0, bytes=R * 4 + R * 8 + (2 * E + 1) * 4 + ((T * H * a + T * rowb(H)) if fp8 else 0)),
        "gemm1_swiglu": dict(flops=4 * R * H * F,
                             bytes=T * rowb(H) + R * 4 + Ea * wbytes(H, 2 * F) + R * rowb(F) + (E + 1) * 4),
        "gemm2": dict(flops=2 * R * F * H, bytes=R * rowb(F) + Ea * wbytes(F, H) + R * H * a + (E + 1) * 4),
        "shared_expert": dict(flops=6 * T * H * Fs,
                              bytes=(T * rowb(H) + wbytes(H, 2 * Fs) + wbytes(Fs, H) + 2 * T * rowb(Fs) + T * H * a)
                              if sh else 0),
        "combine": dict(flops=0, bytes=R * H * a + R * 8 + T * H * a + (T * H * a if sh else 0)),
        "active_flops": 2 * T * H * E + 6 * R * H * F + 6 * T * H * Fs,
    }


def cpu_baseline(cfg, d, sample_tokens, min_seconds=10.0):
    """The float64 oracle (as it stands) on the first `sample_tokens` tokens of the same layer.

    Expert weights are copied to the host one expert at a time when the oracle asks for them
    (dequantised by the oracle's own e4m3 decoder for the e4m3 workload); that copy is timed
    apart and left out of the reported rate.
    """
    import torch
    from oracle import e4m3, moe
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    fp8 = cfg.w_dtype == "fp8"
    copy_s = [0.0]

    def weight(w, scales):
        t0 = time.perf_counter()
        if fp8:
            out = e4m3.dequantise_blocks_128x128(w.view(torch.uint8).cpu().numpy(), scales.cpu().numpy())
        else:
            out = w.float().cpu().numpy()
        copy_s[0] += time.perf_counter() - t0
        return out

    x = d["x"][:sample_tokens].float().cpu().numpy()  # bf16 widened exactly
    wr = d["w_router"].cpu().numpy()
    bias = None if d["bias"] is None else d["bias"].cpu().numpy()
    sw1 = sw2 = None
    if cfg.Fs:
        sw1 = weight(d["ws1"], d["ws1_scales"])
        sw2 = weight(d["ws2"], d["ws2_scales"])
    copy_s[0] = 0.0
    runs, dt, wall0 = 0, 0.0, time.perf_counter()
    # repeat the sample until >= min_seconds of oracle time (at most 8 runs, and no new run once
    # two minutes of wall time, weight copies and decoding included, have gone by)
    while runs == 0 or (dt < min_seconds and runs < 8 and time.perf_counter() - wall0 < 120.0):
        t0 = time.perf_counter()
        c0 = copy_s[0]
        moe.forward(x, wr, lambda e: weight(d["w1"][e], None if d["w1_scales"] is None else d["w1_scales"][e]),
                    lambda e: weight(d["w2"][e], None if d["w2_scales"] is None else d["w2_scales"][e]),
                    E=cfg.E, k=cfg.k, score=cfg.score, norm=cfg.norm, bias=bias, shared_w1=sw1, shared_w2=sw2,
                    fp8=fp8)
        dt += time.perf_counter() - t0 - (copy_s[0] - c0)
        runs += 1
        print(f"[bench] cpu oracle run {runs}: {dt:.1f} s oracle time so far, {copy_s[0]:.1f} s weight "
              f"copies", file=sys.stderr, flush=True)
    return {"value": runs * sample_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of the same layer, {runs} run(s); float64 oracle {dt:.1f} s "
                      f"wall (+{copy_s[0]:.1f} s copying the experts it used to the host, not counted)"}


BWD_STAGES = ["recompute_u", "dgrad_h", "swiglu_bwd", "wgrad_w2", "dgrad_x", "wgrad_w1", "shared_expert",
              "router_dx"]
BWD_METRIC = "MoE-layer bwd tokens/s at 1 GPU (gradients of x and every weight); % of MFMA / HBM peak"


def algorithmic_backward(cfg, active_experts=None):
    """FLOPs and unique HBM bytes of each stage of moe_backward (u = x W1 recomputed in fp32;
    dh' = dy W2^T fp32; du and g h in the operand dtype; weight gradients fp32)."""
    T, H, E, k, F, Fs = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    R = T * k
    Ea = E if active_experts is None else active_experts
    a = 4 if cfg.act_dtype == "f32" else 2

    def group(rows, tokens, ne, Fg):
        return {
            "recompute_u": dict(flops=4 * rows * H * Fg, bytes=tokens * H * a + ne * H * 2 * Fg * a + rows * 2 * Fg * 4),
            "dgrad_h": dict(flops=2 * rows * Fg * H, bytes=tokens * H * a + ne * Fg * H * a + rows * Fg * 4),
            "swiglu_bwd": dict(flops=0, bytes=rows * 3 * Fg * 4 + rows * 3 * Fg * a + rows * 4),
            "wgrad_w2": dict(flops=2 * rows * Fg * H, bytes=rows * Fg * a + tokens * H * a + ne * Fg * H * 4),
            "dgrad_x": dict(flops=4 * rows * Fg * H, bytes=rows * 2 * Fg * a + ne * H * 2 * Fg * a + rows * H * 4),
            "wgrad_w1": dict(flops=4 * rows * H * Fg, bytes=tokens * H * a + rows * 2 * Fg * a + ne * H * 2 * Fg * 4),
        }
    out = group(R, T, Ea, F)
    sh = group(T, T, 1, Fs) if Fs else None
    out["shared_expert"] = dict(flops=sum(v["flops"] for v in sh.values()) if sh else 0,
                                bytes=sum(v["bytes"] for v in sh.values()) if sh else 0)
    out["router_dx"] = dict(flops=4 * T * H * E,
                            bytes=T * E * 12 + R * 12 + H * E * 8 + T * H * a + R * H * 4 + T * H * 4 * (3 if Fs else 2)
                            + T * H * a)
    out["total_flops"] = sum(out[s]["flops"] for s in BWD_STAGES)
    return out


def cpu_baseline_backward(cfg, d, dy, sample_tokens, min_seconds=10.0):
    """The float64 oracle backward (as it stands) on the first `sample_tokens` tokens of the layer.

    Its forward dict (the routing and the permuted rows the backward consumes) is built by the
    oracle forward first and not timed; expert weights are copied to the host once, untimed."""
    from oracle import backward as obw, moe
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    w1 = [d["w1"][e].float().cpu().numpy() for e in range(cfg.E)]
    w2 = [d["w2"][e].float().cpu().numpy() for e in range(cfg.E)]
    sw1 = d["ws1"].float().cpu().numpy() if cfg.Fs else None
    sw2 = d["ws2"].float().cpu().numpy() if cfg.Fs else None
    copy_s = time.perf_counter() - t0
    x = d["x"][:sample_tokens].float().cpu().numpy()
    g = dy[:sample_tokens].float().cpu().numpy()
    wr = d["w_router"].cpu().numpy()
    bias = None if d["bias"] is None else d["bias"].cpu().numpy()
    fw = moe.forward(x, wr, lambda e: w1[e], lambda e: w2[e], E=cfg.E, k=cfg.k, score=cfg.score, norm=cfg.norm,
                     bias=bias, shared_w1=sw1, shared_w2=sw2)
    runs, dt = 0, 0.0
    while runs == 0 or (dt < min_seconds and runs < 8):
        t0 = time.perf_counter()
        obw.backward(fw, x, wr, lambda e: w1[e], lambda e: w2[e], g, score=cfg.score, norm=cfg.norm,
                     shared_w1=sw1, shared_w2=sw2)
        dt += time.perf_counter() - t0
        runs += 1
        print(f"[bench] cpu oracle backward run {runs}: {dt:.1f} s so far", file=sys.stderr, flush=True)
    return {"value": runs * sample_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of the same layer, {runs} run(s) of the float64 oracle "
                      f"backward, {dt:.1f} s (its forward dict and {copy_s:.1f} s of weight copies not counted)"}


def bench_backward(args, cfg, d, layer, torch, moe_gpu, _lib):
    """Time K calls of moe_backward (one step = the whole layer backward for the batch); the
    routing state comes from one untimed forward, and every input is resident in HBM."""
    import moe_inputs
    dev = "cuda"
    x = d["x"]
    _, dbg = moe_gpu.forward(x, layer, debug=True)
    dy = moe_inputs.make_upstream_grad(cfg, seed=0, device=dev)
    c_layer = layer.c_struct(x.dtype)
    L = _lib.lib()
    need = int(L.moe_backward_workspace_size(ctypes.byref(c_layer), cfg.T))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    f32 = torch.float32
    grads = {"dx": torch.empty_like(x), "dw_router": torch.empty(cfg.H, cfg.E, dtype=f32, device=dev),
             "dw1": torch.empty(cfg.E, cfg.H, 2 * cfg.F, dtype=f32, device=dev),
             "dw2": torch.empty(cfg.E, cfg.F, cfg.H, dtype=f32, device=dev),
             "dws1": torch.empty(cfg.H, 2 * cfg.Fs, dtype=f32, device=dev) if cfg.Fs else None,
             "dws2": torch.empty(cfg.Fs, cfg.H, dtype=f32, device=dev) if cfg.Fs else None}
    r_c = _lib.MoeRoutingC(**{kk: dbg[kk].data_ptr() for kk in moe_gpu.ROUTING_KEYS})
    g_c = _lib.MoeGradsC(**{kk: (None if t is None else t.data_ptr()) for kk, t in grads.items()})
    stream = torch.cuda.current_stream()
    hip = _hip()
    K, W = args.steps, args.warmup
    n_ev = _lib.MOE_NUM_BWD_STAGE_EVENTS
    events = []
    for _ in range(K):
        row = (ctypes.c_void_p * n_ev)()
        for i in range(n_ev):
            ev = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(ev)) == 0
            row[i] = ev.value
        events.append(row)

    def step(ev_row=None):
        _lib.check("moe_backward", L.moe_backward(ctypes.byref(c_layer), ctypes.c_void_p(x.data_ptr()),
                                                  ctypes.c_void_p(dy.data_ptr()), cfg.T, ctypes.byref(r_c),
                                                  ctypes.byref(g_c), ev_row, ctypes.c_void_p(ws.data_ptr()), need,
                                                  ctypes.c_void_p(stream.cuda_stream)))

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    print(f"[bench] backward: {W} warmup steps done", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(K):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] backward: {K} timed steps done: {elapsed * 1e3 / K:.3f} ms/step", file=sys.stderr, flush=True)
    stage_ms = {s: [] for s in BWD_STAGES}
    for row in events:
        for i, s in enumerate(BWD_STAGES):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(row[i]), ctypes.c_void_p(row[i + 1])) == 0
            stage_ms[s].append(ms.value)
        for ev in row:
            hip.hipEventDestroy(ctypes.c_void_p(ev))
    avg_ms = {s: sum(v) / len(v) for s, v in stage_ms.items()}
    active = int((dbg["expert_counts"] > 0).sum().item())
    alg = algorithmic_backward(cfg, active)
    mm_dtype = cfg.act_dtype
    peak_tf = PEAK_TFLOPS[mm_dtype]
    ms_per_step = elapsed * 1e3 / K
    stages = {}
    for s in BWD_STAGES:
        ms = avg_ms[s]
        if ms <= 0 or (alg[s]["flops"] == 0 and alg[s]["bytes"] == 0):
            continue
        rec = {"us": round(ms * 1e3, 2), "GB_s": round(alg[s]["bytes"] / (ms * 1e-3) / 1e9, 1),
               "frac_hbm_peak": round(alg[s]["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if alg[s]["flops"]:
            rec["TFLOP_s"] = round(alg[s]["flops"] / (ms * 1e-3) / 1e12, 1)
            rec["frac_mfma_peak"] = round(rec["TFLOP_s"] / peak_tf, 4)
        stages[s] = rec
    # dominant kernel: the longest single-launch stage among the routed expert GEMMs
    dom = max(["recompute_u", "dgrad_h", "wgrad_w2", "dgrad_x", "wgrad_w1"], key=lambda s: avg_ms[s])
    a_s = alg[dom]
    t_s = avg_ms[dom] * 1e-3
    mfma_bound = a_s["flops"] / (peak_tf * 1e12) >= a_s["bytes"] / (PEAK_HBM_GBS * 1e9)
    layout = {"recompute_u": "NN", "dgrad_h": "NT", "dgrad_x": "NT", "wgrad_w2": "TN", "wgrad_w1": "TN"}[dom]
    if mfma_bound:
        achieved, peak, unit = a_s["flops"] / t_s / 1e12, peak_tf, "TFLOP/s"
    else:
        achieved, peak, unit = a_s["bytes"] / t_s / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"kernel": f"bwd_gemm_kernel<{layout}> ({dom})", "bound": "mfma" if mfma_bound else "hbm",
                "achieved": round(achieved, 1), "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": measured_backward_traffic() if (args.workload == "mixtral_8x7b" and dom == "wgrad_w1")
                else None,
                "flops_per_launch": a_s["flops"], "algorithmic_bytes_per_launch": a_s["bytes"],
                "avg_launch_us": round(avg_ms[dom] * 1e3, 2)}
    out = {
        "metric": BWD_METRIC, "value": round(cfg.T * K / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": mm_dtype, "data": "synthetic",
        "config": {"workload": cfg.description + " -- backward", "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
                   "F": cfg.F, "Fs": cfg.Fs, "experts_with_rows": active, "parallelism": "single GPU"},
        "tflops": round(alg["total_flops"] / (ms_per_step * 1e-3) / 1e12, 1),
        "frac_mfma_peak": round(alg["total_flops"] / (ms_per_step * 1e-3) / 1e12 / peak_tf, 4),
        "stages": stages,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        default_sample = {"mixtral_8x7b": 512, "qwen3_235b": 64, "deepseek_v3": 32, "tiny_fp32": 256}
        out["cpu_baseline"] = cpu_baseline_backward(cfg, d, dy, args.cpu_sample_tokens or
                                                    default_sample.get(args.workload, 64))
    print(json.dumps(out), flush=True)


def practical_ceilings(torch):
    """Same-run context figures (not targets): a 2 GiB device copy and a bf16 8192^3 library matmul."""
    out = {}
    src = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["device_copy_GB_s"] = round(2 * (1 << 31) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    torch.matmul(a, b)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    out["bf16_matmul_8192_TFLOP_s"] = round(2 * 8192 ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    out["note"] = "torch copy_ and torch.matmul (hipBLASLt) on the same GPU in the same run; context only"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_8x7b",
                    help="layer shape: mixtral_8x7b (default), qwen3_235b, deepseek_v3, deepseek_v3_fp8_zipf, tiny_fp32")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens in the CPU oracle sample (default: about 10-30 s of oracle work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the same-run copy / matmul ceilings")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer backward (moe_backward) instead of the forward (bf16 / fp32 workloads)")
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

    cfg = moe_inputs.CONFIGS[args.workload]
    dev = "cuda"
    d = moe_inputs.make_inputs(cfg, seed=0, weight_device=dev, act_device=dev)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    if args.backward:
        bench_backward(args, cfg, d, layer, torch, moe_gpu, _lib)
        return
    print(f"[bench] {args.workload}: inputs ready", file=sys.stderr, flush=True)
    x = d["x"]
    c_layer = layer.c_struct(x.dtype)
    L = _lib.lib()
    need = L.moe_workspace_size(ctypes.byref(c_layer), cfg.T)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    y = torch.empty(cfg.T, cfg.H, dtype=x.dtype, device=dev)
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
    print(f"[bench] {W} warmup + {K} timed steps done: {elapsed * 1e3 / K:.3f} ms/step", file=sys.stderr, flush=True)

    stage_ms = {s: [] for s in STAGES}
    step_ms = []  # first to last stage event of each timed step (GPU time of one layer forward)
    for row in events:
        for i, s in enumerate(STAGES):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), row[i], row[i + 1]) == 0
            stage_ms[s].append(ms.value)
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), row[0], row[len(STAGES)]) == 0
        step_ms.append(ms.value)
    for row in events:
        for ev in row:
            hip.hipEventDestroy(ev)
    avg_ms = {s: sum(v) / len(v) for s, v in stage_ms.items()}
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    dbg = _lib.MoeDebugC()
    dbg.expert_counts = counts.data_ptr()
    _lib.check("moe_forward", L.moe_forward(ctypes.byref(c_layer), ctypes.c_void_p(x.data_ptr()), cfg.T,
                                            ctypes.c_void_p(y.data_ptr()), ctypes.byref(dbg),
                                            ctypes.c_void_p(ws.data_ptr()), need,
                                            ctypes.c_void_p(stream.cuda_stream)))
    torch.cuda.synchronize()
    active = int((counts > 0).sum().item())
    alg = algorithmic(cfg, active)
    ms_per_step = elapsed * 1e3 / K
    tokens_per_s = cfg.T * K / elapsed
    active_tflops = alg["active_flops"] / (ms_per_step * 1e-3) / 1e12
    mm_dtype = "fp8" if cfg.w_dtype == "fp8" else cfg.act_dtype
    peak_tf = PEAK_TFLOPS[mm_dtype]

    stages = {}
    for s in STAGES:
        ms = avg_ms[s]
        if ms <= 0 or (alg[s]["flops"] == 0 and alg[s]["bytes"] == 0):
            continue
        rec = {"us": round(ms * 1e3, 2), "GB_s": round(alg[s]["bytes"] / (ms * 1e-3) / 1e9, 1)}
        if alg[s]["flops"]:
            rec["TFLOP_s"] = round(alg[s]["flops"] / (ms * 1e-3) / 1e12, 1)
        if s.startswith("gemm") or s == "shared_expert":
            rec["frac_mfma_peak"] = round(rec["TFLOP_s"] / peak_tf, 4)
        rec["frac_hbm_peak"] = round(rec["GB_s"] / PEAK_HBM_GBS, 4)
        stages[s] = rec
    # dominant kernel: the first grouped GEMM; its binding roof is the larger of the two ideal times
    g1 = alg["gemm1_swiglu"]
    g1_s = avg_ms["gemm1_swiglu"] * 1e-3
    mfma_bound = g1["flops"] / (peak_tf * 1e12) >= g1["bytes"] / (PEAK_HBM_GBS * 1e9)
    kernel = {"fp8": "gemm_fp8_kernel<swiglu> (grouped e4m3 GEMM1 + fused SwiGLU + 1x128 re-quantisation)",
              "bf16": f"gemm_bf16_kernel<{256 if cfg.T * cfg.k >= 192 * cfg.E else 128}, swiglu> "
                      "(grouped GEMM1 + fused SwiGLU)",
              "f32": "gemm_f32_kernel<swiglu> (grouped fp32 GEMM1 + fused SwiGLU)"}[mm_dtype]
    if mfma_bound:
        achieved, peak, unit = g1["flops"] / g1_s / 1e12, peak_tf, "TFLOP/s"
    else:
        achieved, peak, unit = g1["bytes"] / g1_s / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"kernel": kernel, "bound": "mfma" if mfma_bound else "hbm", "achieved": round(achieved, 1),
                "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": measured_traffic() if args.workload == "mixtral_8x7b" else None,
                "flops_per_launch": g1["flops"], "algorithmic_bytes_per_launch": g1["bytes"],
                "avg_launch_us": round(avg_ms["gemm1_swiglu"] * 1e3, 2)}
    router = f"fp32 {cfg.score} top-{cfg.k}" + (" renormalised" if cfg.norm else "") + \
        (" + Zipf(1.2) selection bias" if cfg.zipf_bias else "")
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": mm_dtype, "data": "synthetic",
        "config": {"workload": cfg.description, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "F": cfg.F,
                   "Fs": cfg.Fs, "router": router, "experts_with_rows": active, "parallelism": "single GPU"},
        "active_tflops": round(active_tflops, 1),
        "frac_mfma_peak": round(active_tflops / peak_tf, 4),
        "stages": stages,
        "roofline": roofline,
    }
    st = sorted(step_ms)
    out["step_gpu_ms"] = {"median": round(st[len(st) // 2], 4), "min": round(st[0], 4),
                          "p90": round(st[min(len(st) - 1, int(0.9 * len(st)))], 4)}
    if not args.no_ceilings:
        out["practical_ceilings"] = practical_ceilings(torch)
    if not args.no_cpu_baseline:
        default_sample = {"mixtral_8x7b": 4096, "qwen3_235b": 256, "deepseek_v3": 128,
                          "deepseek_v3_fp8_zipf": 128, "tiny_fp32": 256}
        out["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_sample_tokens or default_sample[args.workload])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
