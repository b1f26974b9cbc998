"""Parity at the full workload sizes, in the launch configuration the benchmark
times (emeans_train with the scaling-law recipe, seed 1234).

* assign: every row of X is assigned on the GPU; the oracle checks a random
  sample of rows (labels and distances).
* train: lockstep replay of the whole run; the oracle checks a random sample
  of slots per step against its own fp64 assignment, adopts the GPU labels,
  and the final states are compared (running counts bit for bit, revival log
  exactly, centroids to 1e-4 relative L2 for fp32 data and 1e-2 for bf16,
  final MSE on a sample of rows to 1e-3). One step mid-run is checked slot
  by slot: every one of its 65,536 slots (one whole assign launch), and the
  first 262,144 slots of a 4M-row step on the large workload.

The workloads: embedding-like 1M x 768 (k 4096), deep-like 1M x 96 (k 16384),
SIFT-like 1M x 128 (k 16384), fp32, 5 passes; large 100M x 128 bf16
(k 65536), 3 passes, generated on the GPU and read back by the oracle.
"""
import time

import numpy as np
import pytest

import oracle
from mini_means_amd import datagen

from parity import check_dists, check_labels, lockstep, rel_l2

pytestmark = pytest.mark.gpu

FP32 = ["embedding", "deep", "sift"]


def log(msg):
    print(f"[fullsize] {msg}", flush=True)


@pytest.fixture(scope="module")
def mm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mini_means_amd
    mini_means_amd.lib()
    return mini_means_amd


_cache = {}


def workload(name):
    """(host X, device X) of a full-size fp32 workload, generated once."""
    import torch
    if name not in _cache:
        _cache.clear()
        W = datagen.WORKLOADS[name]
        t0 = time.time()
        X = datagen.make(W["gen"], W["n"], W["d"])
        _cache[name] = (X, torch.from_numpy(X).cuda())
        log(f"{name}: generated {X.shape} in {time.time() - t0:.1f}s")
    return _cache[name]


@pytest.mark.parametrize("name", FP32)
def test_fullsize_assign(mm, name):
    import torch
    W = datagen.WORKLOADS[name]
    X, Xd = workload(name)
    rng = np.random.default_rng(7)
    C = np.ascontiguousarray(X[rng.choice(len(X), W["k"], replace=False)])
    lab, dist = mm.assign(Xd, torch.from_numpy(C).cuda())
    lab, dist = lab.cpu().numpy(), dist.cpu().numpy()
    rows = np.sort(rng.choice(len(X), 2048, replace=False))
    olab, d1, d2 = oracle.assign(X, C, rows)
    check_labels(X, C, rows, lab[rows], olab, d1, d2, what=f"{name} assign")
    check_dists(X, C, rows, lab[rows], dist[rows], what=f"{name} assign")
    assert lab.min() >= 0 and lab.max() < W["k"]


@pytest.mark.parametrize("name", FP32)
def test_fullsize_train_lockstep(mm, name):
    import torch
    W = datagen.WORKLOADS[name]
    X, Xd = workload(name)
    k, T, seed = W["k"], W["T"], 1234
    t0 = time.time()
    out = mm.train(Xd, k, T, seed, trace=True, counts=True, split_log_cap=1 << 21)
    torch.cuda.synchronize()
    log(f"{name}: GPU train {time.time() - t0:.2f}s, {out.stats['n_splits']} revivals")
    t0 = time.time()
    mid = oracle.recipe(len(X), X.shape[1], k, T)["total_steps"] // 2
    res, summ = lockstep(X, out, k, T, seed, sample=192, rng_seed=3, progress=16,
                         full={mid: None})
    log(f"{name}: oracle replay {time.time() - t0:.1f}s {summ}")
    assert summ["steps"] == res.recipe["total_steps"]
    assert summ["full_slots"] == res.recipe["batch_size"]
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert out.stats["n_splits"] == len(res.split_log)
    assert out.split_log == [tuple(s) for s in res.split_log]
    assert out.stats["dead_at_end"] == res.dead_at_end
    assert np.array_equal(out.labels.cpu().numpy(), res.labels)
    C = out.centroids.cpu().numpy()
    err = rel_l2(C, res.centroids)
    log(f"{name}: centroid rel L2 {err:.2e}")
    assert err <= 1e-4
    rows = np.sort(np.random.default_rng(5).choice(len(X), 8192, replace=False))
    m_gpu = oracle.mse(X[rows], C)
    m_ref = oracle.mse(X[rows], res.centroids)
    assert abs(m_gpu - m_ref) <= 1e-3 * m_ref
    np.testing.assert_allclose(out.stats["obj"], res.obj, rtol=1e-4)


@pytest.fixture(scope="module")
def large(mm):
    """The large workload on the GPU plus its host read-back (bf16 bits)."""
    import torch
    _cache.clear()
    W = datagen.WORKLOADS["large"]
    t0 = time.time()
    Xd = datagen.large_device(n=W["n"], d=W["d"])
    torch.cuda.synchronize()
    log(f"large: generated {tuple(Xd.shape)} on the GPU in {time.time() - t0:.1f}s")
    t0 = time.time()
    X = np.empty((W["n"], W["d"]), dtype=np.uint16)
    step = 1 << 22
    for lo in range(0, W["n"], step):
        hi = min(W["n"], lo + step)
        X[lo:hi] = Xd[lo:hi].view(torch.int16).cpu().numpy().view(np.uint16)
    log(f"large: read back in {time.time() - t0:.1f}s")
    yield X, Xd
    del Xd
    torch.cuda.empty_cache()


def test_fullsize_large_assign(mm, large):
    import torch
    W = datagen.WORKLOADS["large"]
    X, Xd = large
    rng = np.random.default_rng(9)
    C = np.ascontiguousarray(oracle.to_f32(X[rng.choice(len(X), W["k"], replace=False)]))
    nb = 1 << 22  # one batch of the recipe
    lab, dist = mm.assign(Xd[:nb], torch.from_numpy(C).cuda())
    lab, dist = lab.cpu().numpy(), dist.cpu().numpy()
    rows = np.sort(rng.choice(nb, 1024, replace=False))
    Cs = oracle.bf16_round(C)
    olab, d1, d2 = oracle.assign(X, Cs, rows)
    check_labels(X, Cs, rows, lab[rows], olab, d1, d2, what="large assign")
    check_dists(X, Cs, rows, lab[rows], dist[rows], what="large assign")


def res_mid(k, T):
    W = datagen.WORKLOADS["large"]
    return oracle.recipe(W["n"], W["d"], k, T)["total_steps"] // 2


def test_fullsize_large_train_lockstep(mm, large):
    import torch
    W = datagen.WORKLOADS["large"]
    X, Xd = large
    k, T, seed = W["k"], W["T"], 1234
    t0 = time.time()
    out = mm.train(Xd, k, T, seed, trace=True, counts=True, split_log_cap=1 << 22)
    torch.cuda.synchronize()
    log(f"large: GPU train {time.time() - t0:.2f}s, {out.stats['n_splits']} revivals")
    t0 = time.time()
    res, summ = lockstep(X, out, k, T, seed, sample=96, rng_seed=4, progress=8,
                         full={res_mid(k, T): 1 << 18})
    log(f"large: oracle replay {time.time() - t0:.1f}s {summ}")
    assert summ["full_slots"] == 1 << 18
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert out.split_log == [tuple(s) for s in res.split_log]
    assert np.array_equal(out.labels.cpu().numpy(), res.labels)
    C = out.centroids.cpu().numpy()
    err = rel_l2(C, res.centroids)
    log(f"large: centroid rel L2 {err:.2e}")
    assert err <= 1e-2
    rows = np.sort(np.random.default_rng(6).choice(len(X), 2048, replace=False))
    m_gpu = oracle.mse(X[rows], C)
    m_ref = oracle.mse(X[rows], res.centroids)
    assert abs(m_gpu - m_ref) <= 1e-3 * m_ref
