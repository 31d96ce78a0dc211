"""Write the per-expert routing bias of the skewed-routing DeepSeek-V3-shaped workload.

The workload asks for expert loads that follow a Zipf law with exponent 1.2 and
for some experts to receive no tokens.  Nothing on the pages says how such a bias
is drawn, so this script fixes a recipe and calibrates it with the oracle only:

1. expert e gets Zipf rank r(e) from ``torch.randperm(E)`` seeded with 0 (rank 1 = heaviest);
2. the 16 lowest ranks get target load 0 (bias -1e4: never selected, since k <= E - 16);
3. the others get targets c * r^-1.2, water-filled so they sum to T*k with no expert above T
   (a token selects an expert at most once);
4. b is calibrated on the oracle's fp32 router logits of the workload's seeded x and W_r:
   200 steps of b_e += 0.1 * (ln(target_e + 1) - ln(load_e + 1)), loads from the oracle's
   selection key + top-k + expert counts;
5. b is written as fp32 hex floats, one per line, with the realised loads in the header.

Run from the repository root:  python tests/golden/make_zipf_bias.py
"""

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import moe  # noqa: E402
import moe_inputs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias_deepseek_v3_fp8.txt")
ZIPF_S = 1.2
N_ZERO = 16
STEPS = 200
RATE = 0.1


def zipf_targets(E, T, k, ranks):
    r = ranks.astype(np.float64)
    live = r <= E - N_ZERO
    w = np.where(live, r ** -ZIPF_S, 0.0)
    total = float(T * k)
    sat = np.zeros(E, dtype=bool)
    while True:
        c = (total - T * sat.sum()) / w[~sat].sum()
        tgt = np.where(sat, float(T), c * w)
        over = (tgt > T) & ~sat
        if not over.any():
            return tgt
        sat |= over


def main():
    cfg = moe_inputs.CONFIGS["deepseek_v3_fp8_zipf"]
    T, E, k = cfg.T, cfg.E, cfg.k
    x, w_router = moe_inputs.make_host_inputs(cfg, seed=0)
    logits = moe.router_logits(x.float().numpy(), w_router.numpy())
    ranks = torch.randperm(E, generator=torch.Generator().manual_seed(0)).numpy() + 1
    target = zipf_targets(E, T, k, ranks)
    b = np.where(target > 0, 0.0, -1e4).astype(np.float32)
    live = target > 0
    for _ in range(STEPS):
        load = moe.expert_counts(moe.topk_ids(moe.selection_key(logits, b), k), E)
        step = RATE * (np.log(target + 1) - np.log(load + 1))
        b = np.where(live, b + step, b).astype(np.float32)
    load = moe.expert_counts(moe.topk_ids(moe.selection_key(logits, b), k), E)
    order = np.argsort(ranks)
    rr = ranks[order][2:E - N_ZERO].astype(np.float64)
    ll = load[order][2:E - N_ZERO].astype(np.float64)
    slope = np.polyfit(np.log(rr), np.log(np.maximum(ll, 1)), 1)[0]
    with open(OUT, "w") as f:
        f.write("# routing bias, one fp32 per expert (hex), for the skewed-routing DeepSeek-V3-shaped layer\n")
        f.write(f"# T={T} E={E} k={k} Zipf s={ZIPF_S}; written by tests/golden/make_zipf_bias.py (oracle only)\n")
        f.write(f"# realised loads: max {load.max()}, mean {load.mean():.1f}, zero-load experts {(load == 0).sum()}, "
                f"log-log slope over ranks 3..{E - N_ZERO} = {slope:.3f}\n")
        f.write(f"# loads by rank 1..10: {load[order][:10].tolist()}\n")
        for v in b:
            f.write(float(np.float32(v)).hex() + "\n")
    print(f"wrote {OUT}: max load {load.max()}, zero {int((load == 0).sum())}, slope {slope:.3f}")


if __name__ == "__main__":
    main()
