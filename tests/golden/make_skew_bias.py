"""Writes tests/golden/skew_bias.json: the skewed score-correction bias of the K3-shape
skewed prefill workload (T = 8192 tokens, seed 4, the K3 layer of seed 1).

The workload asks for 90 of the 896 experts to receive about 80% of the assignments and
for a long tail of 1-5 tokens per expert. Reading: the hot share is 0.78-0.82, and at
least half of the 806 cold experts take 1-5 tokens. The bias (k3gen.skew_bias): the 90
hot experts (ids divisible by 10) keep the layer's U(-0.1, 0.1) bias plus beta; the cold
experts' own bias is replaced by an offset that alone decides their rank, 0 for the 270
warm ones (id % 10 in 1..3) and -tail_offset for the 536 tail ones (id % 10 in 4..9).
tail_offset is bisected until the tail experts average 3 tokens (a count near Poisson(3)
then falls in 1-5 about 87% of the time), and for each tail_offset beta is bisected until
the hot share is 0.80; the warm experts take the rest of the cold pairs. Selection uses
the oracle's unbiased scores (oracle.scores_batch) plus the bias, top 16 per token.

Run: python tests/golden/make_skew_bias.py  (uses only oracle/, the generator and numpy)
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import k3gen  # noqa: E402
import oracle  # noqa: E402

HOT_EVERY, TAIL_FROM = 10, 4
T, X_SEED, LAYER_SEED, K = 8192, 4, 1, 16
TAIL_MEAN = 3.0


def route_counts(sc, base, beta, tail_offset):
    bias = k3gen.skew_bias(base, beta, tail_offset, HOT_EVERY, TAIL_FROM).astype(np.float64)
    ch = sc.astype(np.float64) + bias[None, :]
    top = np.argpartition(-ch, K - 1, axis=1)[:, :K]
    return np.bincount(top.ravel(), minlength=sc.shape[1])


def hot_share(counts, hot):
    return counts[hot].sum() / counts.sum()


def main():
    d = k3gen.K3
    dense = k3gen.gen_dense(d, LAYER_SEED)
    x = k3gen.gen_x(d, X_SEED, T)
    print("oracle scores for 8192 tokens ...", flush=True)
    sc = oracle.scores_batch(d, x, dense["w_router"])
    r = np.arange(d.n_experts) % HOT_EVERY
    hot, tail = r == 0, r >= TAIL_FROM
    warm = ~hot & ~tail

    def fit_beta(tail_offset):
        lo, hi = 0.0, 2.0
        for _ in range(30):
            beta = 0.5 * (lo + hi)
            if hot_share(route_counts(sc, dense["bias"], beta, tail_offset), hot) < 0.80:
                lo = beta
            else:
                hi = beta
        return hi

    lo, hi = 0.0, 2.0  # tail offset: larger -> fewer tokens per tail expert
    for _ in range(30):
        tail_offset = 0.5 * (lo + hi)
        beta = fit_beta(tail_offset)
        mean_tail = route_counts(sc, dense["bias"], beta, tail_offset)[tail].mean()
        print(f"tail offset {tail_offset:.5f} beta {beta:.5f}: tail mean {mean_tail:.3f}", flush=True)
        if mean_tail > TAIL_MEAN:
            lo = tail_offset
        else:
            hi = tail_offset
    tail_offset = hi
    beta = fit_beta(tail_offset)
    counts = route_counts(sc, dense["bias"], beta, tail_offset)
    cold = counts[~hot]
    out = {
        "source": "workload statement of the K3-shape skewed prefill (90 of 896 experts take ~80% "
                  "of assignments, long tail of 1-5 tokens); parameters fitted by this script on the "
                  "oracle's routing of T=8192 tokens (x seed 4, attempt 0), layer seed 1",
        "hot_every": HOT_EVERY, "tail_from": TAIL_FROM, "beta": float(beta), "tail_offset": float(tail_offset),
        "hot_share": float(hot_share(counts, hot)),
        "cold_with_1_to_5_tokens": float(np.mean((cold >= 1) & (cold <= 5))),
        "cold_share_with_0_tokens": float(np.mean(cold == 0)),
        "cold_share_with_6_to_50_tokens": float(np.mean((cold >= 6) & (cold <= 50))),
        "cold_share_with_over_50_tokens": float(np.mean(cold > 50)),
        "hot_tokens_mean": float(counts[hot].mean()), "hot_tokens_max": int(counts[hot].max()),
        "warm_tokens_mean": float(counts[warm].mean()), "tail_tokens_mean": float(counts[tail].mean()),
        "cold_tokens_median": float(np.median(cold)), "cold_tokens_max": int(cold.max()),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_bias.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
