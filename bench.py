"""Benchmark: dropless MoE layer forward on one MI355X.

Default workload: the DeepSeek-V3-shaped layer (T=8192 tokens, H=7168, E=256 routed experts,
top-8 sigmoid router in fp32 with normalised gates, SwiGLU F=2048, one shared expert Fs=2048,
bf16 activations and weights), synthetic seeded inputs resident in HBM: the largest of the
layer shapes that fits one GPU.  One step = one full layer forward through the library's fused
entry point (route -> permute -> grouped SwiGLU GEMMs -> shared expert -> combine).
``--workload`` selects another layer shape (Mixtral-8x7B, Qwen3-235B, DeepSeek-V3 with Zipf loads
and e4m3 experts, DeepSeek-V3 with MXFP4 experts, the tiny fp32 layer) for the same measurement;
``--gate-in-expert`` folds the gates into the experts' SwiGLU epilogue.

Measurement:
  * warm-up W steps, then K steps back to back bracketed by torch.cuda.synchronize(): `value`
    (tokens/s) and `ms_per_step` come from this wall-clock interval;
  * K more steps, each preceded (outside its events) by a write of a 1 GiB scratch buffer, so
    every step starts with caches holding other data: the per-stage times (HIP events the library
    records on the compute stream) and the roofline of the dominant kernel (the routed experts'
    first grouped GEMM with the fused SwiGLU epilogue) come from these;
  * the same cold protocol on the stage entry points alone: route, permute writing its permuted
    rows (bf16 copy and e4m3 quantisation) and combine, as HBM GB/s;
  * same-run ceilings: this repository's own streaming-copy kernel on 2 GiB, and the vendor
    library's bf16 8192^3 matmul;
  * the float64 CPU oracle on a bounded sample of the same layer (`cpu_baseline`).
Every measured call is preceded by a marker kernel whose grid size names the phase, so a
rocprofv3 trace of this command can be cut into phases and launch positions
(``--summarize-trace``).

With --backward a step is one call of the layer backward instead (gradients of x and of every
weight for a dy drawn from its own seed, routing state from one untimed forward); the line then
carries the backward's stages and the roofline of its longest expert GEMM.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--backward]
                       [--no-cpu-baseline] [--no-ceilings] [--no-stage-bench]
       python bench.py --summarize-trace DIR [DIR ...]      (rocprofv3 csv output -> markdown)
       python bench.py --copy-calibration                   (copies for scaling HBM counters)
"""

from __future__ import annotations

import argparse
import ctypes
import csv
import glob
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd active TFLOPS + tokens/s at 1 GPU; % of MFMA / HBM peak"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}  # MI355X dense MFMA by operand type
PEAK_BF16_TFLOPS = PEAK_TFLOPS["bf16"]
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
STAGES = ["route", "permute", "gemm1_swiglu", "gemm2", "shared_expert", "combine"]
DEFAULT_WORKLOAD = "deepseek_v3"
FLUSH_BYTES = 1 << 30       # scratch written before every cold repetition
CSRC = os.path.join(ROOT, "mixture_experts_layer_fp32_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

# Phases of a bench run, as the grid size (in workgroups) of the marker launched before every
# measured call; --summarize-trace cuts a rocprofv3 trace at the markers.
PHASES = {1: "forward warm-up", 2: "forward timed (back to back)", 3: "forward cold (1 GiB flush before each)",
          4: "route alone (cold)", 5: "permute + bf16 row copy alone (cold)",
          6: "permute + e4m3 row quantisation alone (cold)", 7: "combine alone (cold)",
          8: "backward warm-up", 9: "backward timed", 10: "copy ceiling (own kernel, 2 GiB)",
          11: "copy calibration (own kernel, 1 GiB)", 12: "untimed set-up work"}
(PH_WARM, PH_TIMED, PH_COLD, PH_ROUTE, PH_PERM, PH_PERM8, PH_COMB, PH_BWARM, PH_BTIMED, PH_CEIL, PH_CAL,
 PH_UNTIMED) = range(1, 13)

# Sources each measured kernel is built from: a counter summary applies to the kernel only while
# these files' code lines (// comments and blank lines removed) hash as they did when it was taken.
GEMM_SOURCES = [os.path.join(CSRC, f) for f in ("gemm.hip", "gemm_common.hpp", "common.hpp")]
FP8_GEMM_SOURCES = [os.path.join(CSRC, f) for f in ("gemm_fp8.hip", "gemm_common.hpp", "common.hpp")]
BWD_SOURCES = [os.path.join(CSRC, f) for f in ("backward.hip", "gemm.hip", "gemm_common.hpp", "common.hpp")]


def code_sha256(files):
    """SHA-256 of the files' code lines: // comments and blank lines removed (a comment edit does
    not change the kernel the counters were taken on)."""
    h = hashlib.sha256()
    for f in files:
        for line in open(f, encoding="utf-8"):
            code = re.sub(r"//.*", "", line).strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def gemm_source_sha256():
    return code_sha256(GEMM_SOURCES)


def backward_source_sha256():
    return code_sha256(BWD_SOURCES)


def tree_sha256():
    """SHA-256 over every library source and header (file names and bytes), in name order."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(INCLUDE, "*.h")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def git_head():
    try:
        out = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        return out.stdout.strip() if out.returncode == 0 and out.stdout.strip() else None
    except Exception:  # no git on the machine, or not a checkout
        return None


def bf16_tile_rows(rows, E):
    """Row height of the bf16 grouped GEMM tiles the library picks for `rows` permuted rows over E
    experts (the rule in gemm.hip: 128 below 192 rows per expert on average, 320 from 232 to 304,
    else 256)."""
    if rows < 192 * E:
        return 128
    return 320 if 232 * E <= rows <= 304 * E else 256


def traffic_file(kernel_tag, workload):
    return os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}_hbm_traffic.txt")


def read_kv(path):
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    return kv


def measured_traffic_from(path, sha_key, sha):
    """HBM bytes per launch from a committed PMC summary, or None when the file is missing or the
    kernel's sources changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    kv = read_kv(path)
    if kv.get(sha_key) != sha or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def measured_traffic(workload, fp8=False):
    """HBM bytes per launch of the routed experts' first grouped GEMM on `workload`."""
    sha = code_sha256(FP8_GEMM_SOURCES if fp8 else GEMM_SOURCES)
    return measured_traffic_from(traffic_file("gemm1_swiglu", workload), "gemm_source_sha256", sha)


def measured_backward_traffic(workload):
    return measured_traffic_from(traffic_file("wgrad_w1_backward", workload), "backward_source_sha256",
                                 backward_source_sha256())


def _hip():
    h = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


class BenchUtil:
    """The measurement helpers of libmoe_bench_util.so: streaming copy, flush fill, phase marker."""

    def __init__(self, torch):
        from mixture_experts_layer_fp32_amd.build import BENCH_UTIL_PATH
        if not os.path.exists(BENCH_UTIL_PATH):
            raise ImportError(f"{BENCH_UTIL_PATH} is missing: build with `python -m mixture_experts_layer_fp32_amd.build`")
        u = ctypes.CDLL(BENCH_UTIL_PATH)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        u.moe_bench_copy.argtypes = [vp, vp, i64, vp]
        u.moe_bench_fill.argtypes = [vp, i64, ctypes.c_uint32, vp]
        u.moe_bench_mark.argtypes = [vp, ctypes.c_int32, ctypes.c_uint32, vp]
        for f in (u.moe_bench_copy, u.moe_bench_fill, u.moe_bench_mark):
            f.restype = ctypes.c_int
        self.u = u
        self.torch = torch
        self.mark_buf = torch.zeros(64, dtype=torch.int32, device="cuda")
        self.flush_buf = None

    def _stream(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    @staticmethod
    def _ok(name, rc):
        if rc != 0:
            raise RuntimeError(f"{name} returned {rc}")

    def mark(self, phase, step=0):
        self._ok("moe_bench_mark", self.u.moe_bench_mark(ctypes.c_void_p(self.mark_buf.data_ptr()), phase, step,
                                                          self._stream()))

    def flush(self):
        if self.flush_buf is None:
            self.flush_buf = self.torch.empty(FLUSH_BYTES, dtype=self.torch.uint8, device="cuda")
        self._ok("moe_bench_fill", self.u.moe_bench_fill(ctypes.c_void_p(self.flush_buf.data_ptr()), FLUSH_BYTES,
                                                          0x3F800000, self._stream()))

    def copy(self, src, dst, nbytes):
        self._ok("moe_bench_copy", self.u.moe_bench_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                                          nbytes, self._stream()))


def algorithmic(cfg, active_experts=None):
    """Useful FLOPs and the bytes each stage of the fused forward must move (unique HBM bytes).

    Activations in the config's dtype (bf16 2 B, fp32 4 B); weights and the permuted / hidden
    rows of the e4m3 path 1 B plus one fp32 scale per 128 values (weights: per 128 x 128 block);
    of the MXFP4 path half a byte plus one E8M0 byte per 32 values.
    Only experts that received rows are streamed (``active_experts``, default all E).
    """
    T, H, E, k, F, Fs = cfg.T, cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    R = T * k
    Ea = E if active_experts is None else active_experts
    fp8 = cfg.w_dtype == "fp8"
    fp4 = cfg.w_dtype == "mxfp4"
    a = 4 if cfg.act_dtype == "f32" else 2
    if fp8:
        rowb = lambda n: n + n // 128 * 4   # noqa: E731 -- one row of n values
        wbytes = lambda K, N: K * N + (K // 128) * (N // 128) * 4  # noqa: E731
    elif fp4:
        rowb = lambda n: n // 2 + n // 32  # noqa: E731
        wbytes = lambda K, N: K * N // 2 + K * N // 32  # noqa: E731
    else:
        rowb = lambda n: n * a  # noqa: E731
        wbytes = lambda K, N: K * N * a  # noqa: E731
    sh = bool(Fs)
    return {
        "route": dict(flops=2 * T * H * E, bytes=T * H * a + H * E * 4 + R * 8 + (E * 4 if cfg.zipf_bias else 0)),
        # the fused forward writes no permuted copy: dispatch = ids -> maps (+ the e4m3 path's
        # per-token quantisation of x), and GEMM1 gathers the token rows it needs
        "permute": dict(flops=0, bytes=R * 4 + R * 8 + (2 * E + 1) * 4 + ((T * H * a + T * rowb(H)) if fp8 or fp4
                                                                          else 0)),
        "gemm1_swiglu": dict(flops=4 * R * H * F,
                             bytes=T * rowb(H) + R * 4 + Ea * wbytes(H, 2 * F) + R * rowb(F) + (E + 1) * 4),
        "gemm2": dict(flops=2 * R * F * H, bytes=R * rowb(F) + Ea * wbytes(F, H) + R * H * a + (E + 1) * 4),
        "shared_expert": dict(flops=6 * T * H * Fs,
                              bytes=(T * rowb(H) + wbytes(H, 2 * Fs) + wbytes(Fs, H) + 2 * T * rowb(Fs) + T * H * a)
                              if sh else 0),
        "combine": dict(flops=0, bytes=R * H * a + R * 8 + T * H * a + (T * H * a if sh else 0)),
        "active_flops": 2 * T * H * E + 6 * R * H * F + 6 * T * H * Fs,
    }


def algorithmic_stage_calls(cfg):
    """Unique HBM bytes of the stage entry points called alone (no logits requested):
    route reads x and W_r and writes ids + gates; permute reads x and the ids and writes the
    permuted rows (bf16 copy, or e4m3 codes + one fp32 scale per 128 values), row_map, src_token,
    counts and offsets; combine reads the permuted expert outputs and gates and writes y."""
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    R = T * k
    a = 4 if cfg.act_dtype == "f32" else 2
    maps = R * 4 + R * 8 + (2 * E + 1) * 4
    return {
        "route": T * H * a + H * E * 4 + R * 8,
        "permute_bf16": T * H * a + R * H * a + maps,
        "permute_e4m3": T * H * a + R * (H + H // 128 * 4) + maps,
        "combine": R * H * a + R * 8 + T * H * a,
    }


def cpu_baseline(cfg, d, sample_tokens, min_seconds=10.0):
    """The float64 oracle (as it stands) on the first `sample_tokens` tokens of the same layer.

    Expert weights are copied to the host one expert at a time when the oracle asks for them
    (dequantised by the oracle's own e4m3 decoder for the e4m3 workload); that copy is timed
    apart and left out of the reported rate.
    """
    import torch
    from oracle import e4m3, moe, mxfp4
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    fp8 = cfg.w_dtype == "fp8"
    fp4 = cfg.w_dtype == "mxfp4"
    copy_s = [0.0]

    def weight(w, scales):
        t0 = time.perf_counter()
        if fp8:
            out = e4m3.dequantise_blocks_128x128(w.view(torch.uint8).cpu().numpy(), scales.cpu().numpy())
        elif fp4:  # stored [N, K/2] codes + [N, K/32] E8M0 -> the logical [K, N]
            out = mxfp4.dequantise_packed(w.view(torch.uint8).cpu().numpy(), scales.view(torch.uint8).cpu().numpy()).T
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
                    fp8=fp8, mxfp4_mode=fp4)
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


def bench_backward(args, cfg, d, layer, torch, moe_gpu, _lib, util):
    """Time K calls of moe_backward (one step = the whole layer backward for the batch); the
    routing state comes from one untimed forward, and every input is resident in HBM."""
    import moe_inputs
    dev = "cuda"
    x = d["x"]
    util.mark(PH_UNTIMED)
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

    for i in range(W):
        util.mark(PH_BWARM, i)
        step()
    torch.cuda.synchronize()
    print(f"[bench] backward: {W} warmup steps done", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(K):
        util.mark(PH_BTIMED, i)
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
    if mm_dtype == "bf16":
        # bf16 expert GEMMs run on the forward's grouped-GEMM kernel (operand mode: 0 weights [K, N],
        # 1 weights [N, K], 2 per-expert products); the weight-gradient stages include the transposes
        grouped = bf16_tile_rows(cfg.T * cfg.k, cfg.E)
        bm = {"recompute_u": grouped, "dgrad_h": grouped, "dgrad_x": grouped,
              "wgrad_w2": 256 if cfg.F >= 256 else 128, "wgrad_w1": 256 if cfg.H >= 256 else 128}[dom]
        mode = {"recompute_u": 0, "dgrad_h": 1, "dgrad_x": 1, "wgrad_w2": 2, "wgrad_w1": 2}[dom]
        out_f32 = "false" if dom == "dgrad_x" else "true"  # dx_perm is written in bf16
        kname = f"gemm_bf16_kernel<{bm}, 2, false, {out_f32}, 1, {mode}> ({dom}" + \
                (", with its operand transpose)" if mode == 2 else ")")
    else:
        layout = {"recompute_u": "NN", "dgrad_h": "NT", "dgrad_x": "NT", "wgrad_w2": "TN", "wgrad_w1": "TN"}[dom]
        kname = f"bwd_gemm_kernel<{layout}> ({dom})"
    if mfma_bound:
        achieved, peak, unit = a_s["flops"] / t_s / 1e12, peak_tf, "TFLOP/s"
    else:
        achieved, peak, unit = a_s["bytes"] / t_s / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"kernel": kname, "bound": "mfma" if mfma_bound else "hbm",
                "achieved": round(achieved, 1), "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": measured_backward_traffic(args.workload) if dom == "wgrad_w1" else None,
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




def stage_bench(cfg, d, layer, torch, moe_gpu, util, reps):
    """The stage entry points alone, each repetition preceded (outside its events) by the 1 GiB
    flush: route (no logits), permute writing the permuted rows (bf16 copy, and e4m3 codes + 1x128
    scales when H % 128 == 0), combine of a permuted expert output.  Returns {name: record}."""
    alg = algorithmic_stage_calls(cfg)
    x = d["x"]
    util.mark(PH_UNTIMED)
    ids, gates = moe_gpu.route(x, layer.w_router, cfg.k, cfg.score, cfg.norm, bias=layer.bias)
    dev = x.device
    calls = [("route", PH_ROUTE, lambda: moe_gpu.route(x, layer.w_router, cfg.k, cfg.score, cfg.norm, bias=layer.bias))]
    if cfg.act_dtype == "bf16":
        calls.append(("permute_bf16", PH_PERM, lambda: moe_gpu.permute(x, ids, cfg.E)))
        if cfg.H % 128 == 0:
            calls.append(("permute_e4m3", PH_PERM8,
                          lambda: moe_gpu.permute(x, ids, cfg.E, perm_dtype=torch.float8_e4m3fn)))
    p = moe_gpu.permute(x, ids, cfg.E, with_rows=False)
    y_perm = torch.empty(cfg.T * cfg.k, cfg.H, dtype=x.dtype, device=dev).normal_()
    calls.append(("combine", PH_COMB, lambda: moe_gpu.unpermute_combine(y_perm, p["row_map"], gates)))
    out = {}
    for name, phase, fn in calls:
        util.mark(PH_UNTIMED)
        fn()  # first call: the caching allocator settles its outputs and workspace
        times = []
        for i in range(reps):
            util.flush()
            util.mark(phase, i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        med = times[len(times) // 2]
        gbs = alg[name] / (med * 1e-3) / 1e9
        out[name] = {"us_median": round(med * 1e3, 2), "us_min": round(times[0] * 1e3, 2),
                     "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": alg[name]}
    del y_perm
    return out


def practical_ceilings(torch, util):
    """Same-run context figures (not targets): this repository's own streaming-copy kernel on a
    2 GiB buffer (bench_util.hip) and the vendor library's bf16 8192^3 matmul."""
    out = {}
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    util.mark(PH_UNTIMED)
    util.copy(src, dst, n)
    torch.cuda.synchronize()
    times = []
    for i in range(5):
        util.mark(PH_CEIL, i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        util.copy(src, dst, n)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    out["own_copy_kernel_GB_s"] = round(2 * n / (min(times) * 1e-3) / 1e9, 1)
    del src, dst
    util.mark(PH_UNTIMED)
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    out["bf16_matmul_8192_TFLOP_s"] = round(2 * 8192 ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    out["note"] = ("own_copy_kernel: best of 5 copies of 2 GiB (reads + writes counted); bf16_matmul: "
                   "torch.matmul (hipBLASLt); same GPU, same run; context only")
    return out


def input_hashes(d, cfg):
    """SHA-256 of the input tensors' bytes: x, w_router, the routing bias, the first and last
    expert's matrices and the shared expert (every expert's bytes would take minutes to copy)."""
    def sha(t):
        if t is None:
            return None
        b = t.detach().contiguous().view(-1).view(__import__("torch").uint8).cpu().numpy().tobytes()
        return hashlib.sha256(b).hexdigest()
    E = cfg.E
    out = {"x": sha(d["x"]), "w_router": sha(d["w_router"]), "bias": sha(d["bias"]),
           "w1[0]": sha(d["w1"][0]), "w2[0]": sha(d["w2"][0]),
           f"w1[{E - 1}]": sha(d["w1"][E - 1]), f"w2[{E - 1}]": sha(d["w2"][E - 1])}
    if cfg.Fs:
        out["ws1"], out["ws2"] = sha(d["ws1"]), sha(d["ws2"])
    if d["w1_scales"] is not None:
        out["w1_scales"], out["w2_scales"] = sha(d["w1_scales"]), sha(d["w2_scales"])
    return {k: v for k, v in out.items() if v is not None}


# ------------------------------------------------------------------------ rocprofv3 summaries
def short_kernel_name(name):
    """'void moe::(anonymous namespace)::gemm_bf16_kernel<256, 2, true, false, 1, 0>(...)' ->
    'gemm_bf16_kernel<256, 2, true, false, 1, 0>'."""
    name = name.strip().strip('"').replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    name = name[:cut]
    depth, last = 0, 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0 and i + 1 < len(name) and name[i + 1] == ":":
            last = i + 2
    return name[last:]


def _field(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    return None


def _dispatches(d):
    """Every dispatch in the rocprofv3 csv files of ONE run (directory `d`): {dispatch id: record}
    with the short kernel name, grid size, duration (ns) and counters (counter collections)."""
    disp = {}
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        for row in csv.DictReader(open(path)):
            i = int(_field(row, "Dispatch_Id", "Correlation_Id"))
            r = disp.setdefault(i, {"counters": {}})
            r["name"] = short_kernel_name(_field(row, "Kernel_Name"))
            r["grid"] = int(float(_field(row, "Grid_Size_X", "Grid_Size") or 0))
            r["ns"] = int(_field(row, "End_Timestamp")) - int(_field(row, "Start_Timestamp"))
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for row in csv.DictReader(open(path)):
            i = int(_field(row, "Dispatch_Id", "Correlation_Id"))
            r = disp.setdefault(i, {"counters": {}})
            r["name"] = short_kernel_name(_field(row, "Kernel_Name"))
            r["grid"] = int(float(_field(row, "Grid_Size", "Grid_Size_X") or 0))
            if _field(row, "End_Timestamp") is not None and "ns" not in r:
                r["ns"] = int(_field(row, "End_Timestamp")) - int(_field(row, "Start_Timestamp"))
            c = _field(row, "Counter_Name")
            r["counters"][c] = r["counters"].get(c, 0.0) + float(_field(row, "Counter_Value"))
    return disp


def all_segments(dirs):
    """segments() of each run directory, concatenated (dispatch ids restart in every run, so runs
    are cut separately and only their steps are pooled)."""
    out = []
    for d in dirs:
        out += segments(_dispatches(d))
    return out


def segments(disp):
    """Cut the dispatches (in dispatch order) at the bench's marker kernels: a list of (phase,
    [(position label, record)]) where the label is 'kernel #n' (its n-th launch in the step).
    The flush fill is left out."""
    segs = []
    for i in sorted(disp):
        r = disp[i]
        name = r.get("name", "?")
        if name.startswith("bench_mark_kernel"):
            segs.append((r["grid"] // 64, []))
            continue
        if name.startswith("fill_kernel") or not segs:
            continue
        if len(name) > 80:  # library kernels of the host framework (input generation, copies)
            name = name[:77] + "..."
        seen = sum(1 for lab, _ in segs[-1][1] if lab.rsplit(" #", 1)[0] == name)
        segs[-1][1].append((f"{name} #{seen}", r))
    return segs


def position_stats(segs, phase, skip=0):
    """{label: [records]} over the steps of `phase` (after skipping its first `skip` steps)."""
    out = {}
    steps = [s for p, s in segs if p == phase][skip:]
    for s in steps:
        for lab, r in s:
            out.setdefault(lab, []).append(r)
    return out, len(steps)


def summarize_trace(dirs):
    """Markdown tables of a rocprofv3 run of bench.py: per phase and launch position, the kernel
    durations (kernel traces) or the average counter values per dispatch (counter collections)."""
    segs = all_segments(dirs)
    lines = []
    for phase in sorted({p for p, _ in segs} - {PH_UNTIMED}):
        stats, nsteps = position_stats(segs, phase)
        lines.append(f"\n### phase {phase}: {PHASES.get(phase, '?')} ({nsteps} steps)\n")
        cnames = sorted({c for rs in stats.values() for r in rs for c in r["counters"]})
        has_t = not cnames and any("ns" in r for rs in stats.values() for r in rs)
        if has_t:
            lines.append("| launch position (kernel #n in the step) | calls | avg us | min us | max us |")
            lines.append("|---|---|---|---|---|")
            total = 0.0
            for lab, rs in stats.items():
                ts = [r["ns"] / 1e3 for r in rs if "ns" in r]
                if not ts:
                    continue
                total += sum(ts) / nsteps
                lines.append(f"| {lab} | {len(ts)} | {sum(ts) / len(ts):.2f} | {min(ts):.2f} | {max(ts):.2f} |")
            lines.append(f"| (sum of the step's kernels, per step) | | {total:.2f} | | |")
        if cnames:
            lines.append("| launch position | calls | " + " | ".join(cnames) + " |")
            lines.append("|---|---|" + "---|" * len(cnames))
            for lab, rs in stats.items():
                vals = []
                for c in cnames:
                    have = [r["counters"][c] for r in rs if c in r["counters"]]
                    vals.append(f"{sum(have) / len(have):.6g}" if have else "")
                lines.append(f"| {lab} | {len(rs)} | " + " | ".join(vals) + " |")
    return "\n".join(lines)


def counter_per_launch(dirs, counter, phase, label):
    """Average of `counter` per dispatch at launch position `label` of `phase`."""
    stats, _ = position_stats(all_segments(dirs), phase)
    rs = [r["counters"][counter] for r in stats.get(label, []) if counter in r["counters"]]
    if not rs:
        raise SystemExit(f"no {counter} values for '{label}' in phase {phase} under {dirs}")
    return sum(rs) / len(rs), len(rs)


def traffic_report(args):
    """The HBM-traffic summary file for one launch position: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, each from a run of its own) scaled by what the same counters read for this
    repository's plain copy kernel of 1 GiB (--copy-calibration)."""
    fdir, wdir, cfdir, cwdir = args.traffic_report
    phase, label = args.traffic_phase, args.traffic_label
    f_kib, nf = counter_per_launch([fdir], "FETCH_SIZE", phase, label)
    w_kib, nw = counter_per_launch([wdir], "WRITE_SIZE", phase, label)
    cf_kib, _ = counter_per_launch([cfdir], "FETCH_SIZE", PH_CAL, "stream_copy_kernel #0")
    cw_kib, _ = counter_per_launch([cwdir], "WRITE_SIZE", PH_CAL, "stream_copy_kernel #0")
    fetch_scale = (1 << 30) / (cf_kib * 1024)
    write_scale = (1 << 30) / (cw_kib * 1024)
    rd = f_kib * 1024 * fetch_scale
    wr = w_kib * 1024 * write_scale
    print(f"fetch_size_kib_per_launch = {f_kib:.1f}\nwrite_size_kib_per_launch = {w_kib:.1f}\n"
          f"launches_averaged = {nf} / {nw}\ncopy_fetch_size_kib = {cf_kib:.1f}\ncopy_write_size_kib = {cw_kib:.1f}\n"
          f"fetch_scale = {fetch_scale:.4f}\nwrite_scale = {write_scale:.4f}\nread_bytes_per_launch = {rd:.0f}\n"
          f"write_bytes_per_launch = {wr:.0f}\ntraffic_bytes_per_launch = {rd + wr:.0f}")
    if args.traffic_alg_bytes:
        print(f"algorithmic_bytes_per_launch = {args.traffic_alg_bytes}\n"
              f"traffic_over_algorithmic = {(rd + wr) / args.traffic_alg_bytes:.3f}")
    print(f"gemm_source_sha256 = {gemm_source_sha256()}\nfp8_gemm_source_sha256 = {code_sha256(FP8_GEMM_SOURCES)}\n"
          f"backward_source_sha256 = {backward_source_sha256()}")


# ------------------------------------------------------------------------ forward bench
def bench_forward(args, cfg, d, layer, torch, _lib, util, moe_gpu):
    print(f"[bench] {args.workload}: inputs ready", file=sys.stderr, flush=True)
    x = d["x"]
    c_layer = layer.c_struct(x.dtype)
    L = _lib.lib()
    need = L.moe_workspace_size(ctypes.byref(c_layer), cfg.T)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.empty(cfg.T, cfg.H, dtype=x.dtype, device="cuda")
    stream = torch.cuda.current_stream()
    hip = _hip()
    K, W = args.steps, args.warmup
    nev = len(STAGES) + 1

    def new_events():
        rows = []
        for _ in range(K):
            row = []
            for _ in range(nev):
                ev = ctypes.c_void_p()
                assert hip.hipEventCreate(ctypes.byref(ev)) == 0
                row.append(ev)
            rows.append(row)
        return rows

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

    def read_events(rows):
        stage_ms = {s: [] for s in STAGES}
        step_ms = []
        for row in rows:
            for i, s in enumerate(STAGES):
                ms = ctypes.c_float()
                assert hip.hipEventElapsedTime(ctypes.byref(ms), row[i], row[i + 1]) == 0
                stage_ms[s].append(ms.value)
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), row[0], row[len(STAGES)]) == 0
            step_ms.append(ms.value)
            for ev in row:
                hip.hipEventDestroy(ev)
        return stage_ms, step_ms

    for i in range(W):
        util.mark(PH_WARM, i)
        step()
    torch.cuda.synchronize()
    # timed: K steps back to back (the contract's wall-clock interval)
    warm_events = new_events()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        util.mark(PH_TIMED, i)
        step(warm_events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] {W} warmup + {K} timed steps done: {elapsed * 1e3 / K:.3f} ms/step", file=sys.stderr, flush=True)
    # cold: K steps, each after a 1 GiB scratch write outside its events
    cold_events = new_events()
    for i in range(K):
        util.flush()
        util.mark(PH_COLD, i)
        step(cold_events[i])
    torch.cuda.synchronize()
    print(f"[bench] {K} cold steps done", file=sys.stderr, flush=True)
    warm_ms, warm_step_ms = read_events(warm_events)
    cold_ms, cold_step_ms = read_events(cold_events)

    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    util.mark(PH_UNTIMED)
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
    mm_dtype = {"fp8": "fp8", "mxfp4": "fp4"}.get(cfg.w_dtype, cfg.act_dtype)
    peak_tf = PEAK_TFLOPS[mm_dtype]

    def stage_records(ms_lists):
        avg_ms = {s: sum(v) / len(v) for s, v in ms_lists.items()}
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
        return stages, avg_ms

    stages, cold_avg = stage_records(cold_ms)
    stages_warm, _ = stage_records(warm_ms)
    # dominant kernel: the routed experts' first grouped GEMM (its cold launches); the binding roof
    # is the larger of its two ideal times
    g1 = alg["gemm1_swiglu"]
    g1_s = cold_avg["gemm1_swiglu"] * 1e-3
    mfma_bound = g1["flops"] / (peak_tf * 1e12) >= g1["bytes"] / (PEAK_HBM_GBS * 1e9)
    kernel = {"fp8": "gemm_fp8_kernel<192, true, false> (grouped e4m3 GEMM1 + fused SwiGLU + 1x128 re-quantisation, "
                     "E8M0 variant; the events include the fp32-scale variant <128, true, false> launched beside it, "
                     "which exits at once when every scale is a power of two)",
              "fp4": "gemm_fp4_kernel<128, true, false> (grouped MXFP4 GEMM1 + fused SwiGLU + 1x32 re-quantisation)",
              "bf16": f"gemm_bf16_kernel<{bf16_tile_rows(cfg.T * cfg.k, cfg.E)}, 2, true, false, 1, 0> "
                      "(routed experts' grouped GEMM1 + fused SwiGLU)",
              "f32": "gemm_f32_kernel<swiglu> (grouped fp32 GEMM1 + fused SwiGLU)"}[mm_dtype]
    if mfma_bound:
        achieved, peak, unit = g1["flops"] / g1_s / 1e12, peak_tf, "TFLOP/s"
    else:
        achieved, peak, unit = g1["bytes"] / g1_s / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"kernel": kernel, "bound": "mfma" if mfma_bound else "hbm", "achieved": round(achieved, 1),
                "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(args.workload, fp8=mm_dtype == "fp8") if mm_dtype != "fp4" else None,
                "flops_per_launch": g1["flops"], "algorithmic_bytes_per_launch": g1["bytes"],
                "avg_launch_us": round(cold_avg["gemm1_swiglu"] * 1e3, 2),
                "timing": f"HIP events around the launch on the compute stream, mean of {K} cold steps "
                          "(1 GiB scratch write before each, outside the events)"}
    if mfma_bound is False:
        roofline["tflop_s"] = round(g1["flops"] / g1_s / 1e12, 1)
        roofline["frac_mfma_peak"] = round(g1["flops"] / g1_s / 1e12 / peak_tf, 4)
    router = f"fp32 {cfg.score} top-{cfg.k}" + (" renormalised" if cfg.norm else "") + \
        (" + Zipf(1.2) selection bias" if cfg.zipf_bias else "")
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": mm_dtype, "data": "synthetic",
        "config": {"workload": cfg.description, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "F": cfg.F,
                   "Fs": cfg.Fs, "router": router, "experts_with_rows": active,
                   "gate": "folded into the SwiGLU epilogue" if layer.gate_in_expert else "applied in combine",
                   "parallelism": "single GPU"},
        "active_tflops": round(active_tflops, 1),
        "frac_mfma_peak": round(active_tflops / peak_tf, 4),
        "stages": stages,
        "stages_back_to_back": stages_warm,
        "roofline": roofline,
    }

    def pct(v):
        st = sorted(v)
        return {"median": round(st[len(st) // 2], 4), "min": round(st[0], 4),
                "p90": round(st[min(len(st) - 1, int(0.9 * len(st)))], 4)}
    out["step_gpu_ms"] = {"back_to_back": pct(warm_step_ms), "cold": pct(cold_step_ms)}
    if not args.no_stage_bench:
        out["stage_calls_cold"] = stage_bench(cfg, d, layer, torch, moe_gpu, util, max(5, K // 2))
        print("[bench] stage entry points timed", file=sys.stderr, flush=True)
    if not args.no_ceilings:
        out["practical_ceilings"] = practical_ceilings(torch, util)
        print("[bench] ceilings timed", file=sys.stderr, flush=True)
    out["provenance"] = {"library_source_sha256": tree_sha256(), "git_head": git_head(),
                         "input_sha256": input_hashes(d, cfg), "seed": 0}
    if not args.no_cpu_baseline:
        default_sample = {"mixtral_8x7b": 4096, "qwen3_235b": 256, "deepseek_v3": 128,
                          "deepseek_v3_fp8_zipf": 128, "deepseek_v3_mxfp4": 128, "tiny_fp32": 256}
        out["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_sample_tokens or default_sample[args.workload])
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="layer shape: deepseek_v3 (default), mixtral_8x7b, qwen3_235b, deepseek_v3_fp8_zipf, "
                         "deepseek_v3_mxfp4, tiny_fp32")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens in the CPU oracle sample (default: about 10-30 s of oracle work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the same-run copy / matmul ceilings")
    ap.add_argument("--no-stage-bench", action="store_true", help="skip timing the stage entry points alone")
    ap.add_argument("--gate-in-expert", action="store_true",
                    help="fold the routing gate into the experts' SwiGLU epilogue (combine sums unweighted)")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer backward (moe_backward) instead of the forward (bf16 / fp32 workloads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run this repository's copy kernel on 1 GiB (for scaling HBM counters) and exit")
    ap.add_argument("--summarize-trace", nargs="+", metavar="DIR",
                    help="print per-phase, per-launch-position tables of rocprofv3 csv output under DIR(s)")
    ap.add_argument("--traffic-report", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="HBM traffic summary of one launch position from FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--traffic-phase", type=int, default=PH_COLD)
    ap.add_argument("--traffic-label", default="gemm_bf16_kernel<320, 2, true, false, 1, 0> #0")
    ap.add_argument("--traffic-alg-bytes", type=int, default=0)
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.traffic_report:
        traffic_report(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    util = BenchUtil(torch)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for i in range(args.steps):
            util.mark(PH_CAL, i)
            util.copy(src, dst, 1 << 30)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": 1 << 30, "launches": args.steps}))
        return
    import moe_inputs
    import mixture_experts_layer_fp32_amd as moe_gpu
    from mixture_experts_layer_fp32_amd import _lib

    cfg = moe_inputs.CONFIGS[args.workload]
    d = moe_inputs.make_inputs(cfg, seed=0, weight_device="cuda", act_device="cuda")
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm, gate_in_expert=args.gate_in_expert)
    if args.backward:
        bench_backward(args, cfg, d, layer, torch, moe_gpu, _lib, util)
        return
    bench_forward(args, cfg, d, layer, torch, _lib, util, moe_gpu)


if __name__ == "__main__":
    main()
