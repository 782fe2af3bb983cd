"""The synthetic workloads match their statements (CPU only)."""
import numpy as np

import k3gen
import oracle
from tests import _inputs


def test_skewed_workload_parameters_and_sampled_routing():
    """K3-shape skewed prefill: 90 of the 896 experts take about 80% of the pairs and at
    least half of the others take 1-5 tokens (the fitted figures recorded beside the
    parameters), re-checked on 1024 of the workload's tokens routed by the oracle."""
    p = _inputs.skew_params()
    assert 0.78 <= p["hot_share"] <= 0.82 and p["cold_with_1_to_5_tokens"] >= 0.5
    d = k3gen.K3
    dense = _inputs.dense_for(4)
    r = np.arange(d.n_experts) % p["hot_every"]
    hot = r == 0
    assert hot.sum() == 90
    assert np.all(dense["bias"][(r > 0) & (r < p["tail_from"])] == 0.0)
    assert np.all(dense["bias"][r >= p["tail_from"]] == np.float32(-p["tail_offset"]))
    x = k3gen.gen_x(d, 4, 1024)
    idx, _, _ = oracle.route_batch(d, x, dense["w_router"], dense["bias"])
    counts = np.bincount(idx.ravel(), minlength=d.n_experts)
    share = counts[hot].sum() / counts.sum()
    assert 0.76 <= share <= 0.84, share
    # an eighth of the tokens: a tail expert averages 3 / 8 tokens, so most have none
    assert counts[r >= p["tail_from"]].mean() < 1.0
