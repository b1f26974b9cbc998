"""Free-run parity at the full workload sizes: the GPU trains on its own
(emeans_train, seed 1234, the scaling-law recipe, no help from the oracle),
and its final MSE is compared with the oracle's own free run on the same
synthetic rows, stored by tests/golden/make_freerun_targets.py.

The bar is the one for a whole run: final MSE within 1e-3 relative, on the
training rows and on the held-out rows (blog "k-means Reads Your Data 25
Times. Two Would Do.", the MSE of the section on Lloyd's algorithm, taken after
the closing mean of the faiss README's "How the centroid updates work"). The
two runs need not pass through the same labels: a near-tie resolved
differently in fp32 and fp64 sends them onto different trajectories, and the
test asks that both still land on the same loss.

On the embedding-like set (k = 4096 heavily overlapping unit-norm clusters)
the final loss itself is not reproducible to 1e-3: five runs with the same
seed that differ only in the fp32 summation order of the per-cluster sums
end 1.5e-3 (held-out) and 2.0e-3 (train) apart in relative standard
deviation (seeds 1234-1238: 1.8e-3 and 2.1e-3), and the oracle's own free
runs with seeds 1234-1238 (stored beside its seed-1234 target) spread as
much, 1.8e-3 train and 1.4e-3 held-out. That workload is held to 5e-3,
about three of those standard deviations; the deep- and SIFT-like sets
(same-seed spreads below 1e-4) keep 1e-3.

MSE of the GPU's centroids: on the held-out rows by the oracle (fp64 brute
force); on the training rows from the GPU's own assignment of every row (its
distances are checked against the oracle's elsewhere, to 1e-5 of
|x|^2 + |c|^2, far inside this bar), and on a sample of training rows by the
oracle as well.
"""
import json
import os
import time

import numpy as np
import pytest

import oracle
from mini_means_amd import datagen

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
WORKLOADS = ["tiny", "deep", "sift", "embedding"]
MSE_TOL = {"tiny": 1e-3, "deep": 1e-3, "sift": 1e-3, "embedding": 5e-3}


def log(msg):
    print(f"[freerun] {msg}", flush=True)


@pytest.fixture(scope="module")
def mm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mini_means_amd
    mini_means_amd.lib()
    return mini_means_amd


@pytest.mark.parametrize("name", WORKLOADS)
def test_freerun_final_mse_matches_oracle(mm, name):
    import torch
    with open(os.path.join(GOLDEN, f"freerun_{name}.json")) as f:
        g = json.load(f)
    W = datagen.WORKLOADS[name]
    assert (g["n"], g["d"], g["k"], g["T"], g["seed"]) == (W["n"], W["d"], W["k"], W["T"], 1234)
    t0 = time.time()
    X = datagen.make(W["gen"], W["n"], W["d"])
    Xh = datagen.make(W["gen"], W["heldout"], W["d"], split=1)
    Xd = torch.from_numpy(X).cuda()
    log(f"{name}: data in {time.time() - t0:.1f}s")
    t0 = time.time()
    out = mm.train(Xd, W["k"], W["T"], 1234)
    torch.cuda.synchronize()
    st = out.stats
    log(f"{name}: GPU train {time.time() - t0:.2f}s, {st['n_splits']} revivals "
        f"(oracle {g['n_splits']}), dead at end {st['dead_at_end']} (oracle {g['dead_at_end']})")
    assert st["batch_size"] == g["batch_size"]
    assert st["total_steps"] == g["total_steps"]
    C = out.centroids
    _, dist = mm.assign(Xd, C)
    m_gpu = float(dist.double().mean().item())
    Cn = C.cpu().numpy()
    t0 = time.time()
    h_gpu = oracle.mse(Xh, Cn)
    rows = np.sort(np.random.default_rng(11).choice(len(X), min(len(X), 20_000), replace=False))
    m_smp = oracle.mse(X[rows], Cn)
    _, d_rows = mm.assign(Xd[torch.from_numpy(rows).cuda()], C)
    log(f"{name}: oracle held-out MSE of the GPU centroids in {time.time() - t0:.1f}s")
    rel_m = abs(m_gpu - g["train_mse"]) / g["train_mse"]
    rel_h = abs(h_gpu - g["heldout_mse"]) / g["heldout_mse"]
    log(f"{name}: train MSE gpu {m_gpu:.6f} oracle {g['train_mse']:.6f} (rel {rel_m:.2e}); "
        f"held-out gpu {h_gpu:.6f} oracle {g['heldout_mse']:.6f} (rel {rel_h:.2e})")
    # the GPU's own MSE of its centroids agrees with the oracle's on a sample
    assert abs(float(d_rows.double().mean().item()) - m_smp) <= 1e-5 * m_smp
    tol = MSE_TOL[name]
    assert rel_m <= tol, (m_gpu, g["train_mse"])
    assert rel_h <= tol, (h_gpu, g["heldout_mse"])
    np.testing.assert_allclose(st["obj"][-1], g["obj_per_pass"][-1], rtol=tol)


@pytest.mark.parametrize("name", ["embedding", "deep", "sift"])
def test_gpu_lloyd25_matches_oracle_target(mm, name):
    """The baseline e-means is timed against: 25 Lloyd iterations on the GPU
    (its own labels, Faiss-style splits of empty clusters) end at the
    held-out MSE of the oracle's own Lloyd-25 run from the same starting rows
    (tests/golden/lloyd25_<workload>.json), to the same relative bar as the
    free run, and split as many empty clusters."""
    import torch
    with open(os.path.join(GOLDEN, f"lloyd25_{name}.json")) as f:
        g = json.load(f)
    W = datagen.WORKLOADS[name]
    assert (g["n"], g["d"], g["k"], g["iters"], g["seed"]) == (W["n"], W["d"], W["k"], 25, 1234)
    X = datagen.make(W["gen"], W["n"], W["d"])
    Xh = datagen.make(W["gen"], W["heldout"], W["d"], split=1)
    t0 = time.time()
    out = mm.train(torch.from_numpy(X).cuda(), W["k"], 25.0, 1234, lloyd=True)
    torch.cuda.synchronize()
    log(f"lloyd25 {name}: GPU {time.time() - t0:.2f}s, {out.stats['n_splits']} splits "
        f"(oracle {g.get('empty_cluster_splits', 'not recorded')})")
    if "empty_cluster_splits" not in g and out.stats["n_splits"] > 0:
        # a target stored without a record of its splits was written by plain
        # Lloyd; it equals the splitting Lloyd's only where no cluster empties
        pytest.skip(f"the stored {name} target predates the empty-cluster splits and this run "
                    f"split {out.stats['n_splits']} clusters: rewrite it with "
                    f"tests/golden/make_lloyd_targets.py")
    h_gpu = oracle.mse(Xh, out.centroids.cpu().numpy())
    rel = abs(h_gpu - g["heldout_mse"]) / g["heldout_mse"]
    log(f"lloyd25 {name}: held-out gpu {h_gpu:.6f} oracle {g['heldout_mse']:.6f} (rel {rel:.2e})")
    assert rel <= MSE_TOL[name]
    np.testing.assert_allclose(out.stats["obj"], g["train_mse_history"], rtol=MSE_TOL[name])
    if "empty_cluster_splits" in g:
        ns = g["empty_cluster_splits"]
        assert abs(out.stats["n_splits"] - ns) <= max(5, 0.1 * ns)
