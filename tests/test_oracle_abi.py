"""The oracle's host-pointer mirrors of the library's boundary
(emeans_ref_recipe, emeans_ref_assign, emeans_ref_train in
oracle/emeans_ref.c) take the same steps as the Python oracle, whose own
pins are in test_oracle_pins.py: they must give the same recipe, the same
labels and distances, and the same run bit for bit. CPU only."""
import numpy as np
import pytest

import oracle
from mini_means_amd import datagen

SHAPES = [(10_000, 16, 64, 5.0), (1_000_000, 768, 4096, 5.0), (1_000_000, 96, 16384, 5.0),
          (1_000_000, 128, 16384, 5.0), (100_000_000, 128, 65536, 3.0), (5_003, 37, 77, 1.5),
          (3, 2, 1, 0.5), (1_000, 2, 10, 2.25)]


@pytest.mark.parametrize("n,d,k,T", SHAPES)
def test_abi_recipe_matches_oracle(n, d, k, T):
    a = oracle.abi_recipe(n, d, k, T)
    r = oracle.recipe(n, d, k, T)
    assert a["batch_size"] == r["batch_size"]
    assert a["alpha0"] == r["alpha0"]
    assert a["passes"] == len(r["epoch_rows"])
    assert a["total_steps"] == r["total_steps"]
    assert a["unused_threshold"] == r["unused_threshold"]


def test_abi_assign_matches_oracle():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((700, 24)).astype(np.float32)
    C = rng.standard_normal((53, 24)).astype(np.float32)
    C[10] = C[3]  # an exact tie: the lower index wins
    lab, dist = oracle.abi_assign(X, C)
    olab, d1, _ = oracle.assign(X, C)
    assert np.array_equal(lab, olab)
    assert np.array_equal(dist, d1.astype(np.float32))
    assert not np.any(lab == 10)


def test_abi_train_matches_oracle_run():
    X = datagen.make("tiny", 2_000, 8, seed=3)
    k, T, seed = 40, 2.5, 1234
    C, lab, ns = oracle.abi_train(X, k, T, seed)
    res = oracle.train(X, k, T, seed)
    assert ns == len(res.split_log) and ns > 0  # the run revives clusters
    assert np.array_equal(C, res.centroids)
    assert np.array_equal(lab, res.labels)


def test_abi_rejects_bad_arguments():
    X = np.zeros((10, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.abi_train(X, 11, 1.0)   # k > n
    with pytest.raises(ValueError):
        oracle.abi_train(X, 2, 0.0)    # T <= 0
    with pytest.raises(ValueError):
        oracle.abi_recipe(10, 0, 2, 1.0)
