"""Choose the scale alpha of the log-Zipf expert bias (workload shaping only).

The DeepSeek-R1-shaped layer asks for router logits with a Zipf(s=1.1)
per-expert bias such that the p95 max/mean expert-load ratio is about 4.  A
literal -s*ln(rank) bias gives a far larger skew, so the bias is scaled by
alpha.  This script routes the seeded layer with the CPU oracle over S steps
(each step reseeds the activations) for a few alpha values and prints the p95
skew of each; the chosen value is frozen as ZIPF_ALPHA in workloads/configs.py.
It also reports the K3-shaped decode layer's touched-expert count at that
alpha.  Run: python -m workloads.calibrate_zipf
"""
from __future__ import annotations

import argparse
import sys

import numpy as np

import oracle
from workloads import DEEPSEEK_R1_SHAPED, K3_SHAPED_DECODE, generator as gen


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--alphas", default="0.15,0.2,0.22,0.25,0.28,0.3")
    args = ap.parse_args(argv)
    cfg = DEEPSEEK_R1_SHAPED
    alphas = [float(a) for a in args.alphas.split(",")]
    wg = gen.gate_weight(cfg)
    unit = gen.zipf_bias(cfg.with_(zipf_alpha=1.0))          # -s*ln(rank), alpha = 1
    skews = {a: [] for a in alphas}
    for step in range(args.steps):
        lg = oracle.gate_logits(gen.activations(cfg, step), wg)   # exact, no bias
        for a in alphas:
            scores = (lg + a * unit.astype(np.float64)[None, :]).astype(np.float32)
            ids = oracle.topk_ids(scores, cfg.k)
            skews[a].append(oracle.load_skew(oracle.expert_counts(ids, cfg.E), cfg.T, cfg.k))
        print(f"step {step} done", file=sys.stderr, flush=True)
    for a in alphas:
        print(f"alpha={a:.3f} p95_skew={oracle.p95_nearest_rank(skews[a]):.3f} "
              f"mean_skew={np.mean(skews[a]):.3f}")
    dc = K3_SHAPED_DECODE
    for a in alphas:
        scores = oracle.router_scores(gen.drawn_logits(dc), gen.zipf_bias(dc.with_(zipf_alpha=a)))
        c = oracle.expert_counts(oracle.topk_ids(scores, dc.k), dc.E)
        print(f"decode alpha={a:.3f} touched={int((c > 0).sum())}/{dc.E} max_rows={int(c.max())} "
              f"skew={oracle.load_skew(c, dc.T, dc.k):.2f}")


if __name__ == "__main__":
    main()
