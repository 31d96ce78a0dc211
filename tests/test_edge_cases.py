"""GPU edge cases: tiny and degenerate shapes, forced routings, ties, canaries, graphs."""

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import moe
from tests.checks import check_permutation, max_row_rel, rel_frobenius
from tests.gpu_oracle import TOL, TOL_GATES, TOL_LOGITS, host, routing_from_logits, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_and_check(cfg, seed=0):
    d = moe_inputs.make_inputs(cfg, seed=seed, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    y, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    torch.cuda.synchronize()
    w1 = [weights_of(d["w1"], None, e) for e in range(cfg.E)]
    w2 = [weights_of(d["w2"], None, e) for e in range(cfg.E)]
    sw1 = weights_of(d["ws1"], None, None) if cfg.Fs else None
    sw2 = weights_of(d["ws2"], None, None) if cfg.Fs else None
    o = moe.forward(host(d["x"]), host(d["w_router"]), lambda e: w1[e], lambda e: w2[e], E=cfg.E, k=cfg.k,
                    score=cfg.score, norm=cfg.norm, shared_w1=sw1, shared_w2=sw2, logits=host(dbg["logits"]))
    assert np.array_equal(host(dbg["topk_ids"]), o["ids"])
    assert np.array_equal(host(dbg["row_map"]), o["row_map"])
    return rel_frobenius(host(y), o["y"]), d, dbg, y


@pytest.mark.parametrize("T", [1, 2, 63, 65])
def test_few_tokens(T):
    cfg = moe_inputs.CONFIGS["deepseek_v3"].replace(T=T, H=256, E=16, k=4, F=128, Fs=128)
    err, *_ = _run_and_check(cfg)
    assert err <= TOL["bf16"]


def test_api_maxima():
    """MOE_MAX_EXPERTS experts and MOE_MAX_TOPK slots: full top-k lanes (8 keys per lane), the
    largest expert prefix in LDS, the dense-GEMM router with 3 x 512 columns, the generic combine."""
    cfg = moe_inputs.CONFIGS["deepseek_v3"].replace(T=300, H=256, E=512, k=16, F=128, Fs=0)
    err, d, dbg, _ = _run_and_check(cfg)
    assert err <= TOL["bf16"]
    assert int(host(dbg["expert_counts"]).sum()) == cfg.T * cfg.k


# the H-sliced few-expert kernel, the fused route kernel, the MFMA logits kernel with 16-expert
# column tiles (E = 40) and with 64-expert tiles (E = 64 with H % 64 != 0: not the router GEMM)
@pytest.mark.parametrize("T,E", [(300, 8), (3200, 8), (300, 40), (300, 64)])
def test_route_h_not_a_multiple_of_32(T, E):
    """H = 264 = 8 x 32 + 8: the last 32-wide k-step of the router kernels holds a single 8-element
    chunk.  Logits to the fp32 tolerance, ids bit-exact and gates given those logits."""
    cfg = moe_inputs.CONFIGS["mixtral_8x7b"].replace(T=T, H=264, E=E, F=128)
    d = moe_inputs.make_inputs(cfg, seed=3, weight_device=DEV, act_device=DEV)
    ids, gates, logits = moe_gpu.route(d["x"], d["w_router"], cfg.k, cfg.score, cfg.norm, d["bias"],
                                       return_logits=True)
    torch.cuda.synchronize()
    ref = moe.router_logits(host(d["x"]), host(d["w_router"]))
    assert rel_frobenius(host(logits), ref) <= TOL_LOGITS
    r = routing_from_logits(logits, d["bias"], cfg.k, cfg.score, cfg.norm, cfg.E)
    assert np.array_equal(host(ids), r["ids"])
    assert rel_frobenius(host(gates), r["gates"]) <= TOL_GATES


@pytest.mark.parametrize("E", [70, 130])
def test_route_fp32_many_experts(E):
    """fp32 activations with >= 64 experts: the fp32 FMA logits kernel's 64-expert tiles, the last
    one partial (70, 130 = 2 x 64 + 2).  The logits are exact fp32 dot products up to summation
    order: logits to the fp32 tolerance, ids bit-exact and gates given those logits."""
    cfg = moe_inputs.CONFIGS["tiny_fp32"].replace(T=300, H=160, E=E, k=6, F=128)
    d = moe_inputs.make_inputs(cfg, seed=4, weight_device=DEV, act_device=DEV)
    assert d["x"].dtype == torch.float32
    ids, gates, logits = moe_gpu.route(d["x"], d["w_router"], cfg.k, cfg.score, cfg.norm, d["bias"],
                                       return_logits=True)
    torch.cuda.synchronize()
    ref = moe.router_logits(host(d["x"]), host(d["w_router"]))
    assert rel_frobenius(host(logits), ref) <= TOL_LOGITS
    r = routing_from_logits(logits, d["bias"], cfg.k, cfg.score, cfg.norm, cfg.E)
    assert np.array_equal(host(ids), r["ids"])
    assert rel_frobenius(host(gates), r["gates"]) <= TOL_GATES


def test_k_equals_E():
    cfg = moe_inputs.CONFIGS["qwen3_235b"].replace(T=130, H=128, E=6, k=6, F=128)
    err, d, dbg, _ = _run_and_check(cfg)
    assert err <= TOL["bf16"]
    assert (host(dbg["expert_counts"]) == 130).all()


def test_fp32_tiny_against_tolerance():
    err, *_ = _run_and_check(moe_inputs.CONFIGS["tiny_fp32"].replace(T=33))
    assert err <= TOL["f32"]


def test_forced_routing_one_expert_takes_all_and_empty_experts():
    """Caller-supplied ids (router replay): experts 3 and 5 get every token, the others none."""
    cfg = moe_inputs.CONFIGS["mixtral_8x7b"].replace(T=777, H=256, E=8, k=2, F=256)
    d = moe_inputs.make_inputs(cfg, seed=3, weight_device=DEV, act_device=DEV)
    ids = torch.tensor([[5, 3]], dtype=torch.int32, device=DEV).repeat(cfg.T, 1)
    p = moe_gpu.permute(d["x"], ids, cfg.E)
    yp = moe_gpu.grouped_swiglu(p["x_perm"], p["offsets"], d["w1"], d["w2"])
    torch.cuda.synchronize()
    cnt = host(p["counts"])
    assert cnt.tolist() == [0, 0, 0, 777, 0, 777, 0, 0]
    check_permutation(host(ids), cnt, host(p["offsets"]), host(p["row_map"]), host(p["src_token"]))
    x = host(d["x"])
    ref3 = moe.swiglu_expert(x, weights_of(d["w1"], None, 3), weights_of(d["w2"], None, 3))
    ref5 = moe.swiglu_expert(x, weights_of(d["w1"], None, 5), weights_of(d["w2"], None, 5))
    got = host(yp)
    assert rel_frobenius(got[:777], ref3) <= TOL["bf16"]
    assert rel_frobenius(got[777:], ref5) <= TOL["bf16"]


def test_tie_heavy_router_is_bit_exact():
    """Integer-valued x and W_r in {-1,0,1}/8: logits are exact, so the GPU logits equal the
    oracle's and the many exact ties must break to the lower expert index in both."""
    cfg = moe_inputs.CONFIGS["qwen3_235b"].replace(T=1000, H=512)
    x, w = moe_inputs.tie_heavy_router(cfg)
    ids, gates, logits = moe_gpu.route(x.to(DEV), w.to(DEV), cfg.k, cfg.score, cfg.norm, return_logits=True)
    torch.cuda.synchronize()
    lo = moe.router_logits(host(x), host(w))
    assert np.array_equal(host(logits), lo)
    ref = moe.topk_ids(lo, cfg.k)
    assert np.array_equal(host(ids), ref)
    ties = sum(len(np.unique(row)) < len(row) for row in lo)
    assert ties > 900  # the case really is tie-heavy


def test_empty_input():
    cfg = moe_inputs.CONFIGS["mixtral_8x7b"].replace(T=4, H=128, F=128)
    d = moe_inputs.make_inputs(cfg, seed=0, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    y = moe_gpu.forward(d["x"][:0], layer)
    assert y.shape == (0, 128)


def test_guard_bands_untouched():
    """Every stage output lives inside a larger buffer filled with a sentinel; only the output
    region may change."""
    cfg = moe_inputs.CONFIGS["deepseek_v3"].replace(T=301, H=256, E=16, k=4, F=128, Fs=0)
    d = moe_inputs.make_inputs(cfg, seed=1, weight_device=DEV, act_device=DEV)
    pad = 4096

    def guarded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * pad,), -7, dtype=torch.int32 if dtype == torch.int32 else torch.float32,
                         device=DEV)
        view = buf[pad:pad + n].view(*shape)
        if dtype not in (torch.int32, torch.float32):
            raise ValueError(dtype)
        return buf, view

    ids_b, ids = guarded((cfg.T, cfg.k), torch.int32)
    g_b, gates = guarded((cfg.T, cfg.k), torch.float32)
    lg_b, logits = guarded((cfg.T, cfg.E), torch.float32)
    from mixture_experts_layer_fp32_amd import _lib
    import ctypes
    L = _lib.lib()
    wsb = L.moe_route_workspace_size(cfg.T, cfg.H, cfg.E, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    st = L.moe_route(ctypes.c_void_p(d["x"].data_ptr()), 1, ctypes.c_void_p(d["w_router"].data_ptr()), None,
                     cfg.T, cfg.H, cfg.E, cfg.k, 1, 1, ctypes.c_void_p(logits.data_ptr()),
                     ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(gates.data_ptr()),
                     ctypes.c_void_p(ws.data_ptr()), wsb, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    for buf in (ids_b, g_b, lg_b):
        h = buf.cpu()
        sentinel = torch.full((pad,), -7, dtype=h.dtype)
        assert torch.equal(h[:pad], sentinel) and torch.equal(h[-pad:], sentinel)
    p = moe_gpu.permute(d["x"], ids, cfg.E)
    R = cfg.T * cfg.k
    xp_b = torch.full((R * cfg.H + 2 * pad,), 12345, dtype=torch.int16, device=DEV)
    xp = xp_b[pad:pad + R * cfg.H].view(torch.bfloat16).view(R, cfg.H)
    yp_b = torch.full((R * cfg.H + 2 * pad,), 12345, dtype=torch.int16, device=DEV)
    yp = yp_b[pad:pad + R * cfg.H].view(torch.bfloat16).view(R, cfg.H)
    L.moe_permute(ctypes.c_void_p(d["x"].data_ptr()), 1, ctypes.c_void_p(ids.data_ptr()), cfg.T, cfg.H, cfg.E,
                  cfg.k, ctypes.c_void_p(xp.data_ptr()), 1, None, ctypes.c_void_p(p["row_map"].data_ptr()),
                  ctypes.c_void_p(p["src_token"].data_ptr()), None, ctypes.c_void_p(p["offsets"].data_ptr()),
                  ctypes.c_void_p(torch.empty(L.moe_permute_workspace_size(cfg.T, cfg.E, cfg.k), dtype=torch.uint8,
                                              device=DEV).data_ptr()),
                  L.moe_permute_workspace_size(cfg.T, cfg.E, cfg.k),
                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    gws = L.moe_grouped_swiglu_workspace_size(R, cfg.F, 1)
    gw = torch.empty(gws, dtype=torch.uint8, device=DEV)
    st = L.moe_grouped_swiglu(ctypes.c_void_p(xp.data_ptr()), None, 1, ctypes.c_void_p(p["offsets"].data_ptr()), R,
                              cfg.E, cfg.H, cfg.F, ctypes.c_void_p(d["w1"].data_ptr()), None,
                              ctypes.c_void_p(d["w2"].data_ptr()), None, ctypes.c_void_p(yp.data_ptr()), 1,
                              ctypes.c_void_p(gw.data_ptr()), gws,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    for buf in (xp_b, yp_b):
        h = buf.cpu()
        sentinel = torch.full((pad,), 12345, dtype=torch.int16)
        assert torch.equal(h[:pad], sentinel) and torch.equal(h[-pad:], sentinel)
    assert not (yp.view(torch.int16) == 12345).all(dim=1).any()  # every row was written


@pytest.mark.parametrize("w_dtype", ["bf16", "e4m3"])
def test_hip_graph_capture_and_replay(w_dtype):
    """The fused forward records into a HIP graph (no sync, no allocation inside) and every
    replay, with eager work in between, reproduces the eager result bit for bit (in e4m3 the
    graph also holds the scale check that picks the GEMM variant)."""
    base = "deepseek_v3" if w_dtype == "bf16" else "deepseek_v3_fp8_zipf"
    cfg = moe_inputs.CONFIGS[base].replace(T=512, H=256, E=16, k=4, F=128, Fs=128)
    if w_dtype == "e4m3":
        cfg = cfg.replace(zipf_bias=False)
    d = moe_inputs.make_inputs(cfg, seed=2, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    ws = torch.empty(moe_gpu.workspace_size(layer, cfg.T, d["x"].dtype), dtype=torch.uint8, device=DEV)
    x = d["x"].clone()
    eager = moe_gpu.forward(x, layer, workspace=ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe_gpu.forward(x, layer, workspace=ws)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_g = moe_gpu.forward(x, layer, workspace=ws)
    for rep in range(3):
        junk = torch.randn(1000, 1000, device=DEV) @ torch.randn(1000, 1000, device=DEV)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        del junk


def test_out_of_range_ids_are_taken_as_expert_zero():
    """Caller-supplied ids outside [0, E) (negative, E, huge) stay in bounds: they are routed to
    expert 0, exactly as the oracle's permutation of the same ids with those entries set to 0."""
    T, H, E, k = 300, 256, 8, 2
    rng = np.random.default_rng(7)
    ids = np.stack([rng.integers(1, E, T), rng.integers(1, E, T)], axis=1).astype(np.int32)
    ids[ids[:, 0] == ids[:, 1], 1] = (ids[ids[:, 0] == ids[:, 1], 0] % (E - 1)) + 1  # distinct per token
    bad = rng.random(T) < 0.3
    ids[bad, 1] = rng.choice(np.array([-1, E, 1 << 20, -(1 << 30)], dtype=np.int32), int(bad.sum()))
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    p = moe_gpu.permute(x, torch.from_numpy(ids).to(DEV), E)
    torch.cuda.synchronize()
    fixed = np.where((ids >= 0) & (ids < E), ids, 0)
    assert (fixed[:, 0] != fixed[:, 1]).all()
    cnt = moe.expert_counts(fixed, E)
    off = moe.expert_offsets(cnt)
    row_map, src = moe.permutation(fixed)
    assert np.array_equal(host(p["counts"]), cnt) and np.array_equal(host(p["offsets"]), off)
    assert np.array_equal(host(p["row_map"]), row_map) and np.array_equal(host(p["src_token"]), src)
    assert np.array_equal(host(p["x_perm"]), host(x)[src])


def test_offsets_past_rows_are_clamped():
    """expert_offsets ending past `rows` (a broken contract) stay in bounds: each expert's range is
    clamped into [0, rows], so expert 1 here covers rows 120..299 of the 300."""
    rows, H, F, E = 300, 256, 256, 2
    gen = torch.Generator().manual_seed(11)
    x = (torch.randn(rows, H, generator=gen)).to(torch.bfloat16).to(DEV)
    w1 = (torch.randn(E, H, 2 * F, generator=gen) * H ** -0.5).to(torch.bfloat16).to(DEV)
    w2 = (torch.randn(E, F, H, generator=gen) * F ** -0.5).to(torch.bfloat16).to(DEV)
    off = torch.tensor([0, 120, 1000], dtype=torch.int32, device=DEV)
    yp = moe_gpu.grouped_swiglu(x, off, w1, w2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = moe.grouped_experts(host(x), np.array([0, 120, rows]), lambda e: host(w1[e]), lambda e: host(w2[e]))
    assert rel_frobenius(host(yp), ref) <= TOL["bf16"]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_320_row_tiles(out_dtype):
    """Experts averaging 192-288 rows take 320-row tiles: one m-tile for experts of up to 320 rows
    (300 and 215 here: 10 and 7 live 32-row blocks), two for 330 rows; the second GEMM stages its
    output per row group (bf16) or per 32-row block (fp32).  H = 640 leaves a half N tile."""
    counts = [300, 215, 330]
    rows, H, F, E = sum(counts), 640, 384, 3
    gen = torch.Generator().manual_seed(13)
    x = (torch.randn(rows, H, generator=gen)).to(torch.bfloat16).to(DEV)
    w1 = (torch.randn(E, H, 2 * F, generator=gen) * H ** -0.5).to(torch.bfloat16).to(DEV)
    w2 = (torch.randn(E, F, H, generator=gen) * F ** -0.5).to(torch.bfloat16).to(DEV)
    off_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    off = torch.from_numpy(off_h).to(DEV)
    yp = moe_gpu.grouped_swiglu(x, off, w1, w2, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = moe.grouped_experts(host(x), off_h.astype(np.int64), lambda e: host(w1[e]), lambda e: host(w2[e]))
    got = host(yp)
    print(f"[edge] 320-row tiles {out_dtype}: rel {rel_frobenius(got, ref):.3e} worst row {max_row_rel(got, ref):.3e}",
          flush=True)
    assert rel_frobenius(got, ref) <= TOL["bf16"] and max_row_rel(got, ref) <= TOL["bf16"]


def test_row_map_outside_range_reads_row_zero():
    """row_map entries outside [0, T k) are read as row 0 by the combine (in bounds)."""
    T, k, H = 50, 4, 128
    gen = torch.Generator().manual_seed(12)
    yp = torch.randn(T * k, H, generator=gen).to(DEV)
    rm = torch.randperm(T * k, generator=gen).reshape(T, k).to(torch.int32)
    rm[3, 1], rm[7, 0], rm[9, 3] = -1, T * k, 1 << 30
    g = torch.rand(T, k, generator=gen)
    y = moe_gpu.unpermute_combine(yp, rm.to(DEV), g.to(DEV))
    torch.cuda.synchronize()
    fixed = torch.where((rm >= 0) & (rm < T * k), rm, torch.zeros_like(rm))
    ref = moe.combine(host(yp), fixed.numpy(), g.numpy().astype(np.float64))
    assert rel_frobenius(host(y), ref) <= TOL["f32"]


def _guarded(n_bytes, pad=4096):
    """A byte buffer with `pad` sentinel bytes (0xA5) on each side of an n_bytes region (16-byte
    aligned: pad is a multiple of 16)."""
    buf = torch.full((n_bytes + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
    return buf, buf[pad:pad + n_bytes]


def _bands_intact(buf, pad=4096):
    h = buf.cpu()
    return bool((h[:pad] == 0xA5).all() and (h[-pad:] == 0xA5).all())


@pytest.mark.parametrize("w_dtype", ["bf16", "e4m3"])
def test_forward_outputs_stay_inside_their_buffers(w_dtype):
    """moe_forward writes y and every requested intermediate only inside their own extent: each
    lives in a buffer with sentinel bytes before and after, which must be untouched; y must also
    match the oracle (so the call did write it)."""
    import ctypes
    from mixture_experts_layer_fp32_amd import _lib
    base = "deepseek_v3" if w_dtype == "bf16" else "deepseek_v3_fp8_zipf"
    cfg = moe_inputs.CONFIGS[base].replace(T=301, H=384, E=16, k=4, F=256, Fs=128, zipf_bias=False)
    d = moe_inputs.make_inputs(cfg, seed=2, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    R = T * k
    fp8 = w_dtype == "e4m3"
    sizes = {"y": T * H * 2, "logits": T * E * 4, "topk_ids": R * 4, "topk_gates": R * 4, "expert_counts": E * 4,
             "expert_offsets": (E + 1) * 4, "row_map": R * 4, "src_token": R * 4,
             "x_perm": R * H * (1 if fp8 else 2), "y_perm": R * H * 2}
    if fp8:
        sizes["x_perm_scales"] = R * (H // 128) * 4
    bufs = {n: _guarded(s) for n, s in sizes.items()}
    dbg = _lib.MoeDebugC(**{n: bufs[n][1].data_ptr() for n in sizes if n != "y"})
    c = layer.c_struct(torch.bfloat16)
    L = _lib.lib()
    need = int(L.moe_workspace_size(ctypes.byref(c), T))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    st = L.moe_forward(ctypes.byref(c), ctypes.c_void_p(d["x"].data_ptr()), T, ctypes.c_void_p(bufs["y"][1].data_ptr()),
                       ctypes.byref(dbg), ctypes.c_void_p(ws.data_ptr()), need,
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    for n, (buf, _) in bufs.items():
        assert _bands_intact(buf), f"{n} written outside its extent"
    y = bufs["y"][1].view(torch.bfloat16).view(T, H)
    y_ref = moe_gpu.forward(d["x"], layer)
    assert torch.equal(y, y_ref)


def test_backward_outputs_stay_inside_their_buffers():
    """moe_backward writes dx and every weight gradient only inside their own extent (sentinel
    bytes on both sides of each, untouched), and the result equals an unguarded call's."""
    cfg = moe_inputs.CONFIGS["deepseek_v3"].replace(T=150, H=320, E=8, k=4, F=256, Fs=128)
    d = moe_inputs.make_inputs(cfg, seed=4, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm)
    T, H, E, F, Fs = cfg.T, cfg.H, cfg.E, cfg.F, cfg.Fs
    _, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    dy = moe_inputs.make_upstream_grad(cfg, seed=4, device=DEV)
    ref = moe_gpu.backward(d["x"], dy, layer, dbg)
    import ctypes
    from mixture_experts_layer_fp32_amd import _lib
    sizes = {"dx": T * H * 2, "dw_router": H * E * 4, "dw1": E * H * 2 * F * 4, "dw2": E * F * H * 4,
             "dws1": H * 2 * Fs * 4, "dws2": Fs * H * 4}
    bufs = {n: _guarded(s) for n, s in sizes.items()}
    c = layer.c_struct(torch.bfloat16)
    L = _lib.lib()
    need = int(L.moe_backward_workspace_size(ctypes.byref(c), T))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    r_c = _lib.MoeRoutingC(**{kk: dbg[kk].data_ptr() for kk in moe_gpu.ROUTING_KEYS})
    g_c = _lib.MoeGradsC(**{n: bufs[n][1].data_ptr() for n in sizes})
    st = L.moe_backward(ctypes.byref(c), ctypes.c_void_p(d["x"].data_ptr()), ctypes.c_void_p(dy.data_ptr()), T,
                        ctypes.byref(r_c), ctypes.byref(g_c), None, ctypes.c_void_p(ws.data_ptr()), need,
                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    for n, (buf, _) in bufs.items():
        assert _bands_intact(buf), f"{n} written outside its extent"
    assert torch.equal(bufs["dx"][1].view(torch.bfloat16).view(T, H), ref["dx"])
    for n in ("dw_router", "dw1", "dw2", "dws1", "dws2"):
        assert torch.equal(bufs[n][1].view(torch.float32).view(ref[n].shape), ref[n]), n
