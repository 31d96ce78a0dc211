"""Helpers for the GPU parity tests: host copies and oracle evaluations driven by GPU outputs.

Nothing here computes the layer: every number comes from ``oracle`` (CPU, float64) or is a
plain copy of a GPU tensor.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import e4m3, moe, mxfp4

# max relative Frobenius error of floating outputs vs the oracle, by compute dtype (MXFP4: the
# oracle quantises h like the kernels, so the bar covers accumulation-order flips of h codes)
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "mxfp4": 2e-2}
TOL_LOGITS = 1e-5
TOL_GATES = 1e-5


def host(t: torch.Tensor) -> np.ndarray:
    """Exact host copy: bf16 widened to fp32, fp8 kept as uint8 codes, ints as int64."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    if t.dtype in (torch.float8_e4m3fn, torch.float4_e2m1fn_x2, torch.float8_e8m0fnu):
        return t.view(torch.uint8).cpu().numpy()
    if t.dtype in (torch.int32, torch.int64):
        return t.cpu().numpy().astype(np.int64)
    return t.cpu().numpy()


def weights_of(w: torch.Tensor, scales: torch.Tensor | None, e: int | None):
    """float64 host copy of weight matrix e as the logical [K, N] matrix (dequantised for fp8 from
    codes and 128x128 scales; for MXFP4 from the contraction-contiguous [N, K/2] codes and
    [N, K/32] E8M0 scales, transposed)."""
    we = w if e is None else w[e]
    if we.dtype == torch.float8_e4m3fn:
        se = scales if e is None else scales[e]
        return e4m3.dequantise_blocks_128x128(host(we), host(se))
    if we.dtype == torch.float4_e2m1fn_x2:
        se = scales if e is None else scales[e]
        return mxfp4.dequantise_packed(host(we), host(se)).T
    return host(we).astype(np.float64)


def routing_from_logits(logits_gpu, bias, k, score, norm, E):
    """Oracle route + dispatch driven by the GPU's fp32 logits (bit-exact comparison basis)."""
    lg = host(logits_gpu)
    key = moe.selection_key(lg, None if bias is None else host(bias))
    ids = moe.topk_ids(key, k)
    g = moe.gates(lg, ids, score, norm)
    cnt = moe.expert_counts(ids, E)
    off = moe.expert_offsets(cnt)
    row_map, src = moe.permutation(ids)
    return dict(ids=ids, gates=g, counts=cnt, offsets=off, row_map=row_map, src_token=src)
