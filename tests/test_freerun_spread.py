"""The oracle's own seed-to-seed spread of the final loss on the
embedding-like set (1M x 768, k = 4096, T = 5), from its stored free runs
with seeds 1234-1238 (tests/golden/freerun_embedding*.json, written by
make_freerun_targets.py from the oracle alone).

The free-run parity test holds that set to a relative bar of 5e-3 instead of
1e-3 (blog "k-means Reads Your Data 25 Times. Two Would Do.", the MSE of the
section on Lloyd's algorithm): the update is chaotic, and one near-tie
settled the other way sends a run onto another trajectory. This test keeps
the bar tied to the measured spread: it must be at least twice the larger
relative standard deviation over the five seeds, and 1e-3 must not be.
"""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SEEDS = (1234, 1235, 1236, 1237, 1238)
EMBEDDING_BAR = 5e-3


def _runs():
    out = []
    for s in SEEDS:
        name = "freerun_embedding.json" if s == 1234 else f"freerun_embedding_s{s}.json"
        with open(os.path.join(GOLDEN, name)) as fh:
            g = json.load(fh)
        assert g["seed"] == s and g["workload"] == "embedding" and g["T"] == 5.0
        assert g["n"] == 1_000_000 and g["d"] == 768 and g["k"] == 4096
        out.append(g)
    return out


def test_oracle_seed_spread_matches_the_bar():
    runs = _runs()
    tr = np.array([g["train_mse"] for g in runs])
    ho = np.array([g["heldout_mse"] for g in runs])
    rs_tr, rs_ho = tr.std() / tr.mean(), ho.std() / ho.mean()
    spread = max(rs_tr, rs_ho)
    # the seeds give distinct trajectories, each ending near the same loss
    assert len(set(np.round(tr, 12))) == len(SEEDS)
    assert 1e-4 < spread < EMBEDDING_BAR / 2
    assert spread > 1e-3  # a 1e-3 bar would be inside the oracle's own spread
    # held-out loss above training loss on every run (the rows it never saw)
    assert np.all(ho > tr)
