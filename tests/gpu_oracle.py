"""Helpers for the GPU parity tests: host copies and oracle evaluations driven by GPU outputs.

Nothing here computes the layer: every number comes from ``oracle`` (CPU, float64) or is a
plain copy of a GPU tensor.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import e4m3, moe

# max relative Frobenius error of floating outputs vs the oracle, by compute dtype
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
TOL_LOGITS = 1e-5
TOL_GATES = 1e-5


def host(t: torch.Tensor) -> np.ndarray:
    """Exact host copy: bf16 widened to fp32, fp8 kept as uint8 codes, ints as int64."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    if t.dtype in (torch.int32, torch.int64):
        return t.cpu().numpy().astype(np.int64)
    return t.cpu().numpy()


def weights_of(w: torch.Tensor, scales: torch.Tensor | None, e: int | None):
    """float64 host copy of weight matrix e (dequantised for fp8 from codes and 128x128 scales)."""
    we = w if e is None else w[e]
    if we.dtype == torch.float8_e4m3fn:
        se = scales if e is None else scales[e]
        return e4m3.dequantise_blocks_128x128(host(we), host(se))
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
