"""GPU parity of the gate-folded forward (moe_layer.gate_in_expert = 1): the routing gate applied
in the first GEMM's SwiGLU epilogue (h of each permuted row scaled by its gate before rounding),
combine an unweighted sum of the k rows, against the oracle's folded form (reading R9: the same
layer in exact arithmetic; where h is quantised, in MXFP4, the quantiser sees g h).  y and the
gate-weighted expert rows it exposes (moe_debug.y_perm) are held to the layer's bars (relative
Frobenius and worst row: 1e-5 fp32, 2e-2 bf16, 6e-2 e4m3 against the oracle on the dequantised
operands, 2e-2 / 6e-2 MXFP4); the routing and permutation stay bit-exact.
"""

import numpy as np
import pytest
import torch

import moe_inputs
import mixture_experts_layer_fp32_amd as moe_gpu
from oracle import moe
from tests.checks import max_row_rel, rel_frobenius
from tests.gpu_oracle import TOL, host, weights_of

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    "fp32_ragged": moe_inputs.CONFIGS["tiny_fp32"].replace(T=97, E=6, k=3, H=96, F=160),
    "bf16_deepseek_small": moe_inputs.CONFIGS["deepseek_v3"].replace(T=257, H=512, E=32, k=8, F=256, Fs=384),
    "bf16_bm320": moe_inputs.CONFIGS["deepseek_v3"].replace(T=520, H=384, E=8, k=4, F=256, Fs=256),
    "bf16_mixtral_bigtile": moe_inputs.CONFIGS["mixtral_8x7b"].replace(T=1700, H=320, E=3, k=2, F=384),
    "e4m3_small": moe_inputs.CONFIGS["deepseek_v3_fp8_zipf"].replace(T=300, H=640, E=16, k=4, F=384, Fs=256,
                                                                      zipf_bias=False),
    "mxfp4_small": moe_inputs.CONFIGS["deepseek_v3_mxfp4"].replace(T=300, H=512, E=16, k=4, F=256, Fs=256),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gate_folded_forward_matches_oracle(name):
    cfg = CASES[name]
    print(f"[gate-folded] {name}: {cfg}", flush=True)
    d = moe_inputs.make_inputs(cfg, seed=7, weight_device=DEV, act_device=DEV)
    layer = moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm, gate_in_expert=True)
    y, dbg = moe_gpu.forward(d["x"], layer, debug=True)
    plain = moe_gpu.forward(d["x"], moe_gpu.Layer.from_inputs(d, cfg.k, cfg.score, cfg.norm))
    torch.cuda.synchronize()
    fp8 = cfg.w_dtype == "fp8"
    fp4 = cfg.w_dtype == "mxfp4"
    w1 = [weights_of(d["w1"], d["w1_scales"], e) for e in range(cfg.E)]
    w2 = [weights_of(d["w2"], d["w2_scales"], e) for e in range(cfg.E)]
    sw1 = weights_of(d["ws1"], d["ws1_scales"], None) if cfg.Fs else None
    sw2 = weights_of(d["ws2"], d["ws2_scales"], None) if cfg.Fs else None
    o = moe.forward(host(d["x"]), host(d["w_router"]), lambda e: w1[e], lambda e: w2[e], E=cfg.E, k=cfg.k,
                    score=cfg.score, norm=cfg.norm, shared_w1=sw1, shared_w2=sw2, fp8=fp8, mxfp4_mode=fp4,
                    logits=host(dbg["logits"]), gate_in_expert=True)
    for key, ref in (("topk_ids", "ids"), ("row_map", "row_map"), ("src_token", "src_token"),
                     ("expert_offsets", "offsets")):
        assert np.array_equal(host(dbg[key]), o[ref]), key
    tol = TOL["fp8" if fp8 else "mxfp4" if fp4 else cfg.act_dtype]
    tol_row = 6e-2 if fp4 else tol  # MXFP4: a rare h code flip moves one row by a few per cent
    yp_ref = o["y_perm"]  # the gate-weighted rows
    yp = host(dbg["y_perm"])
    e_yp, r_yp = rel_frobenius(yp, yp_ref), max_row_rel(yp, yp_ref)
    e_y, r_y = rel_frobenius(host(y), o["y"]), max_row_rel(host(y), o["y"])
    e_plain = rel_frobenius(host(y), host(plain))
    print(f"[gate-folded] {name}: y_perm (gate-weighted) {e_yp:.2e} worst row {r_yp:.2e}; y {e_y:.2e} worst row "
          f"{r_y:.2e}; vs the gate-in-combine forward {e_plain:.2e}", flush=True)
    assert e_yp <= tol and r_yp <= tol_row
    assert e_y <= tol and r_y <= tol_row
