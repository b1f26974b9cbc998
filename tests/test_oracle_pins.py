"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a library
routine (numpy's Philox, scipy's distance and linear-programming routines), a
brute-force loop written differently, a closed form, an invariant the pages
state, or values the scaling laws give for the named workloads.
"""
import math
import os

import numpy as np
import pytest
from scipy.optimize import linprog
from scipy.spatial.distance import cdist

import oracle
from mini_means_amd import datagen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# random streams
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ctr,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((5, 7, 11, 13), (123, 456)),
    ((2**64 - 2, 2**63, 1, 2**64 - 1), (2**64 - 1, 2**64 - 1)),
    ((999, 3, 2, 4), (1234, 0)),
])
def test_philox_matches_numpy_library(ctr, key):
    """Philox4x64-10 against numpy.random.Philox (which increments the
    counter before generating a block, hence counter - 1)."""
    v = sum(int(w) << (64 * i) for i, w in enumerate(ctr))   # 256-bit counter
    v = (v - 1) % 2**256
    cc = [(v >> (64 * i)) & (2**64 - 1) for i in range(4)]
    bg = np.random.Philox(counter=np.array(cc, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    want = bg.random_raw(4)
    got = oracle.philox4x64(ctr, key)
    assert [int(v) for v in got] == [int(v) for v in want]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 17, 1000, 10007, 65536, 65537])
def test_permutation_is_bijection(n):
    """README 'Data too big for memory': every vector exactly once per pass."""
    for pass_ in (0, 1, 7):
        p = oracle.perm_range(n, 1234, oracle.STREAM_PERM, pass_, 0, n)
        assert np.array_equal(np.sort(p), np.arange(n))


def test_permutation_ranges_compose_and_differ():
    n = 5000
    full = oracle.perm_range(n, 9, oracle.STREAM_PERM, 3, 0, n)
    parts = np.concatenate([oracle.perm_range(n, 9, oracle.STREAM_PERM, 3, s, min(700, n - s))
                            for s in range(0, n, 700)])
    assert np.array_equal(full, parts)
    other = oracle.perm_range(n, 9, oracle.STREAM_PERM, 4, 0, n)
    assert not np.array_equal(full, other)          # a fresh order every pass
    assert np.mean(full == other) < 0.01
    seed2 = oracle.perm_range(n, 10, oracle.STREAM_PERM, 3, 0, n)
    assert not np.array_equal(full, seed2)


def test_permutation_is_not_trivial():
    """Positions and values are uncorrelated (a weak shuffle-quality check)."""
    n = 100_000
    p = oracle.perm_range(n, 1234, oracle.STREAM_PERM, 0, 0, n).astype(np.float64)
    r = np.corrcoef(np.arange(n), p)[0, 1]
    assert abs(r) < 0.02
    # fixed points of a random permutation: Poisson(1)
    assert np.sum(p == np.arange(n)) < 10


def test_uniform_and_signs_are_balanced():
    u = np.array([oracle.uniform01(1234, t, j) for t in range(20) for j in range(50)])
    assert u.min() >= 0 and u.max() < 1
    assert abs(u.mean() - 0.5) < 0.03
    s = oracle.split_signs(1234, 4, 17, 1000)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 0.1


# ---------------------------------------------------------------------------
# exact assignment
# ---------------------------------------------------------------------------

def _python_argmin(X, C):
    """Pure-Python brute force: distance as sum of squared differences, the
    first smallest index wins."""
    labels, best = [], []
    for x in X.tolist():
        bd, bj = math.inf, -1
        for j, c in enumerate(C.tolist()):
            s = 0.0
            for a, b in zip(x, c):
                s += (a - b) * (a - b)
            if s < bd:
                bd, bj = s, j
        labels.append(bj)
        best.append(bd)
    return np.array(labels), np.array(best)


def test_assign_matches_python_bruteforce():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((40, 5)).astype(np.float32)
    C = rng.standard_normal((7, 5)).astype(np.float32)
    lab, d1, d2 = oracle.assign(X, C)
    pl, pd = _python_argmin(X, C)
    assert np.array_equal(lab, pl)
    np.testing.assert_allclose(d1, pd, rtol=1e-13)
    assert np.all(d2 >= d1)


def test_assign_matches_scipy_cdist_and_rows_subset():
    X = datagen.tiny(n=2000, d=16)
    rng = np.random.default_rng(1)
    C = rng.standard_normal((64, 16)).astype(np.float32)
    D = cdist(X.astype(np.float64), C.astype(np.float64), "sqeuclidean")
    lab, d1, d2 = oracle.assign(X, C)
    assert np.array_equal(lab, np.argmin(D, axis=1))
    np.testing.assert_allclose(d1, D.min(axis=1), rtol=1e-12, atol=1e-12)
    Ds = np.sort(D, axis=1)
    np.testing.assert_allclose(d2, Ds[:, 1], rtol=1e-12, atol=1e-12)
    rows = rng.permutation(2000)[:300]
    lab2, d12, _ = oracle.assign(X, C, rows)
    assert np.array_equal(lab2, lab[rows])
    np.testing.assert_array_equal(d12, d1[rows])


def test_assign_ties_go_to_lowest_index():
    X = np.array([[0.0, 0.0], [1.0, 1.0]], dtype=np.float32)
    C = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0], [1.0, 1.0], [1.0, 1.0]], dtype=np.float32)
    lab, d1, d2 = oracle.assign(X, C)
    assert lab.tolist() == [0, 3]
    assert d1[1] == 0.0 and d2[1] == 0.0


def test_assign_bf16_data():
    X = datagen.large_host(500, d=32, m=16)
    Xf = datagen.bf16_bits_to_f32(X)
    C = oracle.bf16_round(np.random.default_rng(2).standard_normal((16, 32)).astype(np.float32) * 0.2)
    D = cdist(Xf.astype(np.float64), C.astype(np.float64), "sqeuclidean")
    lab, d1, _ = oracle.assign(X, C)
    assert np.array_equal(lab, np.argmin(D, axis=1))
    np.testing.assert_allclose(d1, D.min(axis=1), rtol=1e-12, atol=1e-14)


def test_bf16_round_against_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal(10000).astype(np.float32) * 7
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(oracle.bf16_round(x), want)
    assert np.array_equal(datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(x)), want)


def test_group_matches_add_at():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3000, 9)).astype(np.float32)
    rows = rng.permutation(3000)[:1000]
    labels = rng.integers(0, 13, size=1000).astype(np.int32)
    counts, sums = oracle.group(X, rows, labels, 13)
    want = np.zeros((13, 9))
    np.add.at(want, labels, X[rows].astype(np.float64))
    assert np.array_equal(counts, np.bincount(labels, minlength=13))
    np.testing.assert_allclose(sums, want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# recipe: README "Scaling laws" (values the laws give for the five workloads)
# ---------------------------------------------------------------------------

def _golden_recipes():
    import json
    with open(os.path.join(GOLDEN, "recipes.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_recipes(), ids=lambda c: c["name"])
def test_recipe_golden(case):
    r = oracle.recipe(case["n"], case["d"], case["k"], case["T"])
    assert r["batch_size"] == case["batch_size"]
    assert r["law"] == case["law"]
    assert r["alpha0"] == pytest.approx(case["alpha0"], abs=5e-7)
    assert r["steps_per_pass"] == case["steps_per_pass"]
    assert r["total_steps"] == case["total_steps"]


def test_recipe_constraints():
    for n in (10, 1000, 10**5, 10**7):
        for k in (4, 64, 4096):
            for T in (1.0, 2.5, 5.0):
                r = oracle.recipe(n, 64, k, T)
                B = r["batch_size"]
                assert B & (B - 1) == 0                       # a power of two
                assert B <= max(1, n // 2)                    # capped at about n/2
                assert 1e-4 <= r["alpha0"] <= 1.0             # clamp of eq. (3)
                q = oracle.recipe(n, 64, k, T, batch_law=oracle.LAW_QUALITY)
                if B < max(1, n // 2) and q["batch_size"] > 1:
                    assert B == 8 * q["batch_size"]           # "roughly 8x smaller"
                assert sum(r["epoch_rows"]) == int(math.floor(T)) * n + int(math.floor((T - int(T)) * n))


def test_recipe_low_dimension_rules():
    assert oracle.recipe(10**5, 16, 64, 5)["law"] == oracle.LAW_QUALITY
    assert oracle.recipe(10**5, 17, 64, 5)["law"] == oracle.LAW_THROUGHPUT
    assert oracle.recipe(10**5, 2, 64, 5)["unused_threshold"] == 0.0
    assert oracle.recipe(10**5, 3, 64, 5)["unused_threshold"] == 0.1


def test_recipe_manual_batch_rederives_alpha0():
    r = oracle.recipe(10**6, 64, 1024, 5, batch_size=8192)
    assert r["batch_size"] == 8192
    want = 0.8244 * 1024 ** -0.4617 * 8192 ** 0.9003 * (10**6) ** -0.4498 * 5 ** -0.1057
    assert r["alpha0"] == pytest.approx(want, rel=1e-12)
    r2 = oracle.recipe(10**6, 64, 1024, 5, batch_size=8192, alpha0=0.05)
    assert r2["alpha0"] == 0.05


def test_recipe_fractional_passes():
    r = oracle.recipe(1000, 32, 8, 2.5, batch_size=128)
    assert r["epoch_rows"] == [1000, 1000, 500]
    assert r["steps_per_pass"] == [8, 8, 4]


# ---------------------------------------------------------------------------
# cosine schedule: from alpha0 down to a tenth of it
# ---------------------------------------------------------------------------

def test_cosine_endpoints_and_shape():
    a0 = 0.648496
    al = oracle.alphas(a0, 80)
    assert al[0] == np.float32(a0)
    assert al[-1] == pytest.approx(a0 / 10, rel=1e-6)
    assert np.all(np.diff(al) <= 0)
    # cosine shape: symmetric about the middle of [a0/10, a0]
    mid = (a0 + a0 / 10) / 2
    assert al[:40].mean() + al[40:].mean() == pytest.approx(2 * mid, rel=1e-5)
    assert oracle.alphas(0.3, 1)[0] == np.float32(0.3)


# ---------------------------------------------------------------------------
# EMA update
# ---------------------------------------------------------------------------

def test_running_count_closed_form():
    """With fixed labels, N_j = sum_t a_t prod_{t'>t} (1 - a_t') n_j^t."""
    rng = np.random.default_rng(5)
    n, d, k = 512, 4, 6
    X = rng.standard_normal((n, d)).astype(np.float32)
    fixed = rng.integers(0, k, size=n).astype(np.int32)
    res = oracle.train(X, k, 2.0, seed=7, batch_size=64, unused_threshold=0,
                       labels_for_step=lambda t, rows: fixed[rows])
    al = res.alphas.astype(np.float64)
    want = np.zeros(k)
    t = 0
    for e in range(2):
        rows_all = oracle.perm_range(n, 7, oracle.STREAM_PERM, e, 0, n)
        for s in range(8):
            cnt = np.bincount(fixed[rows_all[s * 64:(s + 1) * 64]], minlength=k)
            want = (1 - al[t]) * want + al[t] * cnt
            t += 1
    np.testing.assert_allclose(res.N, want, rtol=2e-6)


def test_one_step_is_lloyd():
    """Whole set as one batch with a step of 1 is exactly one Lloyd iteration
    (README 'How the centroid updates work'; blog, fourth item)."""
    X = datagen.tiny(n=3000, d=16)
    k = 64
    res = oracle.train(X, k, 1.0, seed=11, batch_size=3000, alpha0=1.0, unused_threshold=0,
                       finalize=False)
    assert res.recipe["total_steps"] == 1
    C0 = X[oracle.init_rows(3000, k, 11)].astype(np.float64)
    D = cdist(X.astype(np.float64), C0, "sqeuclidean")
    lab = np.argmin(D, axis=1)
    want = C0.copy()
    for j in range(k):
        if np.any(lab == j):
            want[j] = X[lab == j].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(res.ema_centroids, want, rtol=0, atol=2e-6)
    C1, _ = oracle.lloyd(X, k, 1, seed=11)
    np.testing.assert_allclose(C1, want, rtol=0, atol=2e-6)


def test_lloyd_mse_never_increases():
    X = datagen.tiny(n=4000, d=16, seed=5)
    _, hist = oracle.lloyd(X, 64, 12, seed=3)
    assert all(b <= a * (1 + 1e-12) for a, b in zip(hist, hist[1:]))
    assert hist[-1] < hist[0]


def test_convex_hull_invariant():
    """Without revival, every EMA centroid stays inside the hull spanned by
    all rows it was ever given (blog, on the rejected gradient update)."""
    rng = np.random.default_rng(6)
    X = rng.standard_normal((400, 3)).astype(np.float32)
    k = 6
    record = []
    res = _train_recording(X, k, 3.0, 2, 32, record)
    seen = [set() for _ in range(k)]
    for rows, lab in record:
        for r, j in zip(rows, lab):
            seen[j].add(int(r))
    checked = 0
    for j in range(k):
        if not seen[j]:
            continue
        P = X[sorted(seen[j])].astype(np.float64)
        c = res.ema_centroids[j].astype(np.float64)
        m = len(P)
        A_eq = np.vstack([P.T, np.ones((1, m))])
        b_eq = np.concatenate([c, [1.0]])
        lp = linprog(np.zeros(m), A_eq=A_eq, b_eq=b_eq, bounds=[(0, None)] * m, method="highs")
        assert lp.status == 0, f"centroid {j} outside the hull of its points"
        checked += 1
    assert checked >= k - 1


def _train_recording(X, k, T, seed, B, record):
    """oracle.train with revival off, recording each step's rows and labels.

    The labels are the oracle's own fp64 assignment on the centroids as they
    stand at that step (the search centroids are captured as the oracle
    hands them to its assignment)."""
    holder = {}
    orig = oracle.search_centroids

    def publish(C, Xd):
        holder["C"] = np.array(C, copy=True)
        return orig(C, Xd)

    def labels(t, rows):
        lab, _, _ = oracle.assign(X, holder["C"], rows)
        record.append((rows.copy(), lab.copy()))
        return lab

    oracle.search_centroids = publish
    try:
        return oracle.train(X, k, T, seed=seed, batch_size=B, unused_threshold=0, finalize=False,
                            labels_for_step=labels, check_slots=lambda t, Bt: np.arange(0),
                            check_hook=lambda c: None)
    finally:
        oracle.search_centroids = orig


def test_finalisation_is_exact_mean_of_last_pass():
    """README "How the centroid updates work": after the final pass every
    centroid equals the plain average of the rows that pass gave it; the
    labels returned are that pass's."""
    X = datagen.tiny(n=5000, d=16, seed=9)
    res = oracle.train(X, 64, 3.0, seed=5)
    lab = res.labels
    assert np.all(lab >= 0)
    for j in range(64):
        m = lab == j
        if m.any():
            np.testing.assert_allclose(res.centroids[j], X[m].astype(np.float64).mean(axis=0),
                                       rtol=0, atol=1e-6)
        else:
            assert np.array_equal(res.centroids[j], res.ema_centroids[j])


def _closing_case():
    import json
    with open(os.path.join(GOLDEN, "closing_mean_hand.json")) as f:
        g = json.load(f)
    C = np.array(g["C_ema"], dtype=np.float32)
    batches = [np.array(b, dtype=np.float32) for b in g["batches"]]
    return g, C, batches


def test_final_closing_mean_hand_example():
    """README "Several GPUs", final_closing_mean: a hand-evaluated replay
    (tests/golden/closing_mean_hand.json). With labels, the -1 row is left
    out and the centroid without rows keeps its value; without labels, each
    row first goes to its nearest final EMA centroid (the far row then pulls
    cluster 1)."""
    g, C, batches = _closing_case()
    Cw, lw = oracle.final_closing_mean(batches, C, np.array(g["assignments"]))
    assert np.array_equal(Cw, np.array(g["with_labels"]["centroids"], dtype=np.float32))
    assert lw.tolist() == g["with_labels"]["labels"]
    Cn, ln = oracle.final_closing_mean(batches, C)
    assert np.array_equal(Cn, np.array(g["without_labels"]["centroids"], dtype=np.float32))
    assert ln.tolist() == g["without_labels"]["labels"]
    Cs, ls = oracle.final_closing_mean(batches, C, spherical=True)
    assert ls.tolist() == g["without_labels_spherical"]["labels"]
    m1 = np.array([113.0, 117.0]) / 4.0
    np.testing.assert_allclose(Cs[1], m1 / np.linalg.norm(m1), rtol=1e-7)
    assert np.array_equal(Cs[2], np.array([-1.0, 0.0], dtype=np.float32))
    assert np.array_equal(Cs[0], C[0])
    with pytest.raises(ValueError):
        oracle.final_closing_mean(batches, C, np.array(g["assignments"][:-1]))


def test_final_closing_mean_without_labels_is_a_lloyd_step():
    """Without labels the replay is one Lloyd step from the EMA centroids:
    scipy's vector quantiser (nearest code by Euclidean distance) gives the
    labels and pandas' group-by mean the centroids, whatever the batch cut."""
    import pandas as pd
    from scipy.cluster.vq import vq
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3000, 7)).astype(np.float32)
    C = rng.standard_normal((40, 7)).astype(np.float32)
    code, _ = vq(X.astype(np.float64), C.astype(np.float64))
    means = pd.DataFrame(X.astype(np.float64)).groupby(code).mean()
    want = C.copy()
    want[means.index.values] = means.values.astype(np.float32)
    for cut in ([3000], [1, 999, 2000], [700] * 4 + [200]):
        edges = np.concatenate([[0], np.cumsum(cut)])
        batches = [X[a:b] for a, b in zip(edges[:-1], edges[1:])]
        got, lab = oracle.final_closing_mean(batches, C)
        assert np.array_equal(lab, code.astype(np.int32))
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-6)


def test_final_closing_mean_from_last_pass_labels_is_the_closing_step():
    """Replaying the rows in row order with the labels the last pass saved
    gives the closing mean of the run itself (the exact last-pass mean,
    pinned above), also for a fractional last pass whose unvisited rows carry
    -1."""
    X = datagen.tiny(n=4000, d=16, seed=11)
    res = oracle.train(X, 48, 2.5, seed=3)
    assert np.sum(res.labels < 0) == 2000
    batches = [X[a:a + 512] for a in range(0, 4000, 512)]
    got, lab = oracle.final_closing_mean(batches, res.ema_centroids, res.labels)
    assert np.array_equal(lab, res.labels)
    np.testing.assert_allclose(got, res.centroids, rtol=0, atol=1e-6)


def test_bf16_search_on_bf16_exact_values_is_the_bf16_data_path():
    """README "Data precision": converting fp32 data to bf16 for the search is
    the same search as storing the data in bf16. On fp32 data whose values are
    bf16 numbers the two runs agree bit for bit (the bf16-data path is pinned
    by the assignment and finalisation tests); an fp32 search of the same
    data takes other decisions, so the option is not ignored."""
    Xb = datagen.large_host(20000, d=32, m=64, seed=21)
    Xf = datagen.bf16_bits_to_f32(Xb)
    kw = dict(seed=7, batch_size=2048)
    a = oracle.train(Xb, 64, 2.0, **kw)
    b = oracle.train(Xf, 64, 2.0, bf16_search=True, **kw)
    assert np.array_equal(a.labels, b.labels)
    assert np.array_equal(a.N, b.N)
    assert np.array_equal(a.centroids, b.centroids)
    assert a.split_log == b.split_log
    c = oracle.train(Xf, 64, 2.0, **kw)
    assert not (np.array_equal(c.labels, b.labels) and np.array_equal(c.centroids, b.centroids))


def test_bf16_search_groups_the_fp32_rows():
    """Only the search uses bf16: the closing mean of every centroid is the
    exact mean of the fp32 rows (not of their bf16 roundings) that the last
    pass assigned to it."""
    X = datagen.tiny(n=5000, d=16, seed=9)
    assert not np.array_equal(oracle.bf16_round(X), X)
    res = oracle.train(X, 64, 3.0, seed=5, bf16_search=True)
    lab = res.labels
    assert np.all(lab >= 0)
    for j in range(64):
        m = lab == j
        if m.any():
            np.testing.assert_allclose(res.centroids[j], X[m].astype(np.float64).mean(axis=0),
                                       rtol=0, atol=1e-6)


# ---------------------------------------------------------------------------
# spherical e-means (README "Spherical e-means")
# ---------------------------------------------------------------------------

def _unit(X):
    X = X.astype(np.float64)
    return (X / np.linalg.norm(X, axis=1, keepdims=True)).astype(np.float32)


def test_assign_ip_matches_numpy_argmax():
    """Highest dot product, lowest index on ties (duplicated centroids)."""
    rng = np.random.default_rng(31)
    X = rng.standard_normal((700, 24)).astype(np.float32)
    C = rng.standard_normal((50, 24)).astype(np.float32)
    C[17] = C[5]          # exact tie: index 5 must win
    C[40] = C[33]
    C[3] = 0.0            # a zero centroid scores 0 (by distance it would score |x|^2)
    # numpy, summed over the dimension in order (so that tied centroids give
    # bit-equal scores, which a blocked matrix product need not)
    X64, C64 = X.astype(np.float64), C.astype(np.float64)
    S = np.zeros((len(X), len(C)))
    for t in range(X.shape[1]):
        S += X64[:, t:t + 1] * C64[None, :, t]
    lab, s1, s2 = oracle.assign_ip(X, C)
    assert np.array_equal(lab, np.argmax(S, axis=1))
    np.testing.assert_allclose(s1, S.max(axis=1), rtol=1e-12, atol=1e-12)
    S2 = np.sort(S, axis=1)
    np.testing.assert_allclose(s2, S2[:, -2], rtol=1e-12, atol=1e-12)
    assert not np.any(np.isin(lab, [17, 40]))
    # a zero centroid scores 0: x = (0.2, -0.98) goes to (1, 0) by dot product
    # (0.2 > 0 > -0.66), while by distance the zero centroid would win
    Cz = np.array([[1.0, 0.0], [0.0, 0.0], [0.6, 0.8]], np.float32)
    xz = np.array([[0.2, -0.98], [-1.0, -0.2], [0.3, 0.954]], np.float32)
    lz, sz, _ = oracle.assign_ip(xz, Cz)
    assert lz.tolist() == [0, 1, 2]
    np.testing.assert_allclose(sz, [0.2, 0.0, 0.6 * 0.3 + 0.8 * 0.954], rtol=1e-6)
    assert oracle.assign(xz, Cz)[0].tolist() == [1, 1, 2]
    rows = np.array([3, 699, 0, 350])
    l2, _, _ = oracle.assign_ip(X, C, rows)
    assert np.array_equal(l2, lab[rows])
    np.testing.assert_allclose(oracle.dot_to(X, C, lab), s1, rtol=1e-12, atol=1e-12)


def test_normalize_keeps_zero_rows():
    C = np.array([[3.0, 4.0], [0.0, 0.0], [-1e-20, 0.0]], np.float32)
    N = oracle.normalize(C)
    np.testing.assert_allclose(N[0], [0.6, 0.8], rtol=1e-7)
    assert np.array_equal(N[1], [0.0, 0.0])
    np.testing.assert_allclose(N[2], [-1.0, 0.0])


def test_spherical_one_step_is_spherical_kmeans():
    """B = n, alpha = 1, no revival: one step is one spherical k-means step
    (assign by the highest cosine to the unit-norm starting centroids, then
    each centroid is its cluster's mean rescaled to norm 1); the error
    reported per row is 2 - 2 x cosine on average, i.e. the mean squared
    distance on the sphere."""
    X = _unit(datagen.tiny(n=3000, d=16, seed=4))
    k = 40
    res = oracle.train(X, k, 1.0, seed=9, batch_size=3000, alpha0=1.0, unused_threshold=0,
                       finalize=False, spherical=True)
    C0 = X[oracle.init_rows(3000, k, 9)].astype(np.float64)
    C0 /= np.linalg.norm(C0, axis=1, keepdims=True)
    S = X.astype(np.float64) @ C0.T
    lab = np.argmax(S, axis=1)
    want = C0.copy()
    for j in range(k):
        m = lab == j
        if m.any():
            mu = X[m].astype(np.float64).mean(axis=0)
            want[j] = mu / np.linalg.norm(mu)
    np.testing.assert_allclose(res.centroids, want, rtol=0, atol=2e-6)
    # fp32 unit vectors have norms 1 +- 1e-7, hence the tolerance
    D = cdist(X.astype(np.float64), C0, "sqeuclidean").min(axis=1)
    np.testing.assert_allclose(res.obj[0], D.mean(), rtol=1e-6)
    np.testing.assert_allclose(res.obj[0], np.mean(2.0 - 2.0 * S.max(axis=1)), rtol=1e-6)


def test_spherical_closing_step_is_normalised_mean():
    X = _unit(datagen.deep(n=4000, d=32, seed=6))
    res = oracle.train(X, 50, 2.0, seed=3, batch_size=512, spherical=True)
    lab = res.labels
    nrm = np.linalg.norm(res.centroids.astype(np.float64), axis=1)
    np.testing.assert_allclose(nrm[nrm > 0], 1.0, atol=1e-6)
    for j in range(50):
        m = lab == j
        if m.any():
            mu = X[m].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(res.centroids[j], mu / np.linalg.norm(mu), rtol=0, atol=2e-6)
    # the EMA centroids are unit-norm too (rescaled after every change)
    en = np.linalg.norm(res.ema_centroids.astype(np.float64), axis=1)
    np.testing.assert_allclose(en[en > 0], 1.0, atol=1e-6)


# ---------------------------------------------------------------------------
# int8 codes (README "Data precision", INT8)
# ---------------------------------------------------------------------------

def test_assign_int8_is_exact_integer_argmin():
    """int8 rows against int8-valued centroids: distances are integers, so the
    oracle's fp64 argmin equals numpy's int64 argmin exactly (lowest index on
    ties, which duplicated centroids force)."""
    rng = np.random.default_rng(41)
    X = rng.integers(-127, 128, size=(900, 48)).astype(np.int8)
    C = rng.integers(-127, 128, size=(70, 48)).astype(np.float32)
    C[9] = C[2]
    X[:40] = C[2].astype(np.int8)                    # exact hits on the tied pair
    D = ((X.astype(np.int64)[:, None, :] - C.astype(np.int64)[None, :, :]) ** 2).sum(-1)
    lab, d1, d2 = oracle.assign(X, C)
    assert np.array_equal(lab, np.argmin(D, axis=1))
    assert np.array_equal(d1, D.min(axis=1).astype(np.float64))
    assert np.all(lab[:40] == 2) and not np.any(lab == 9)


def test_int8_calibration_and_codes():
    rng = np.random.default_rng(42)
    S = (rng.standard_normal((5000, 24)) * rng.uniform(0.1, 9.0, 24) + rng.uniform(-5, 5, 24))
    S = S.astype(np.float32)
    shift, scale = oracle.int8_calibrate(S)
    mn, mx = S.min(0).astype(np.float64), S.max(0).astype(np.float64)
    np.testing.assert_allclose(shift, (mn + mx) / 2, rtol=1e-6, atol=1e-6)
    r = np.max(np.maximum(mx - shift, shift - mn))
    assert math.log2(scale) == int(math.log2(scale))          # a power of two
    assert scale * r <= 127.0 < 2.0 * scale * r               # the largest one that fits
    codes = oracle.int8_encode(S, shift, scale)
    assert codes.dtype == np.int8 and codes.min() >= -127 and codes.max() <= 127
    back = oracle.int8_decode(codes, shift, scale)
    assert np.max(np.abs(back.astype(np.float64) - S)) <= 0.5 / scale * (1 + 1e-6)
    # beyond the calibrated range: clamped to the edge
    far = np.full((1, 24), 1e6, np.float32)
    assert np.all(oracle.int8_encode(far, shift, scale) == 127)
    assert np.all(oracle.int8_encode(-far, shift, scale) == -127)
    # a constant sample (radius 0): scale 1, the shift is the value, codes 0
    const = np.full((7, 3), -2.75, np.float32)
    cs, cscale = oracle.int8_calibrate(const)
    assert cscale == 1.0 and np.all(cs == np.float32(-2.75))
    assert np.all(oracle.int8_encode(const, cs, cscale) == 0)
    # a radius of exactly 127 / 2^e gives scale 2^e; one ulp more halves it
    edge = np.array([[-127.0 / 64], [127.0 / 64]], np.float32)
    assert oracle.int8_calibrate(edge)[1] == 64.0
    edge[1, 0] = np.nextafter(edge[1, 0], np.float32(1e9))
    assert oracle.int8_calibrate(edge)[1] == 32.0
    # the search rounds centroids to the nearest code, ties to even, clamped
    C = np.array([[2.5, -0.5, 127.6, -200.0, 3.49, -2.5]], np.float32)
    assert oracle.int8_round(C).tolist() == [[2.0, -0.0, 127.0, -127.0, 3.0, -2.0]]


# FP16 (README "Data precision", FP16)

def test_f16_rounding_and_decode():
    r = oracle.f16_round(np.array([65504.0, 65519.99, 65520.0, -70000.0, 1.0 + 2.0 ** -11,
                                   1.0 + 3 * 2.0 ** -11, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25],
                                  np.float32))
    # the pages: from 65,520 up, fp16 gives infinity without any error
    assert r[0] == 65504.0 and r[1] == 65504.0 and np.isinf(r[2]) and r[3] == -np.inf
    # ties to even: 1 + 2^-11 -> 1; 1 + 3 2^-11 -> 1 + 2^-9; 2^-25 -> 0; 3 2^-25 -> 2^-23
    assert r[4] == 1.0 and r[5] == 1.0 + 2.0 ** -9
    assert r[6] == 2.0 ** -24 and r[7] == 0.0 and r[8] == 2.0 ** -23
    # the C side decodes every finite binary16 pattern to its value (distance to 0)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    X = bits.view(np.float16)
    X = X[np.isfinite(X)].reshape(-1, 1)
    _, d1, _ = oracle.assign(X, np.zeros((1, 1), np.float32))
    assert np.array_equal(d1, X.astype(np.float64).ravel() ** 2)


def test_f16_training_closing_mean_and_search():
    S = datagen.tiny(n=5000, d=16, seed=9).astype(np.float16)
    res = oracle.train(S, 40, 2.0, seed=5)
    Xv = S.astype(np.float64)
    for j in range(40):
        m = res.labels == j
        if m.any():
            np.testing.assert_allclose(res.centroids[j], Xv[m].mean(axis=0), rtol=1e-6, atol=1e-6)
    # the search uses the centroids rounded to fp16: x = 1 against
    # 1 - 1.1 2^-12 and 1 + 1.2 2^-12: as values the first is nearer, but they
    # round to 1 - 2^-11 and to 1 (an exact hit)
    x1 = np.array([[1.0]], np.float16)
    c2 = np.array([[1.0 - 1.1 * 2.0 ** -12], [1.0 + 1.2 * 2.0 ** -12]], np.float32)
    assert oracle.assign(x1, c2)[0].tolist() == [0]
    assert oracle.f16_round(c2).ravel().tolist() == [1.0 - 2.0 ** -11, 1.0]
    assert oracle.assign(x1, oracle.search_centroids(c2, x1))[0].tolist() == [1]


# FP8 E4M3 (README "Data precision", FP8)

def test_e4m3_table_and_rounding_against_brute_force():
    V = oracle.E4M3_VALUES
    # code points fixed by the OCP E4M3 definition (bias 7, subnormals m * 2^-9)
    assert V[0x00] == 0.0 and V[0x01] == 2.0 ** -9 and V[0x07] == 7 * 2.0 ** -9
    assert V[0x08] == 2.0 ** -6 and V[0x38] == 1.0 and V[0x3F] == 1.875 and V[0x40] == 2.0
    assert V[0x7E] == 448.0 and V[0xB8] == -1.0 and V[0xFE] == -448.0
    assert np.isnan(V[0x7F]) and np.isnan(V[0xFF])
    assert np.all(np.diff(V[:0x7F].astype(np.float64)) > 0)   # codes 0..126 increase
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    finite = V[codes].astype(np.float64)
    rng = np.random.default_rng(7)
    pos = np.sort(V[:0x7F].astype(np.float64))
    mids = (pos[1:] + pos[:-1]) / 2.0                  # exact ties between neighbours
    x = np.concatenate([rng.uniform(-500, 500, 4000),
                        np.exp(rng.uniform(-12, 6, 3000)) * rng.choice([-1, 1], 3000),
                        mids, -mids, [448.0, 455.9, 464.0, 1e6, -1e6, 0.0]]).astype(np.float32)
    got = oracle.e4m3_round(x).astype(np.float64)
    dist = np.abs(x.astype(np.float64)[:, None] - finite[None, :])
    best = dist.min(axis=1, keepdims=True)
    tied = dist == best
    even = tied & ((codes[None, :] & 1) == 0)     # ties go to the even mantissa
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(tied, axis=1))
    assert np.array_equal(got, finite[pick])
    # bit patterns round-trip (all finite codes but -0)
    nz = codes[codes != 0x80]
    assert np.array_equal(oracle.e4m3_bits(V[nz]), nz.astype(np.uint8))


def test_fp8_calibration_and_codes():
    rng = np.random.default_rng(43)
    S = (rng.standard_normal((4000, 20)) * rng.uniform(0.1, 9.0, 20) + rng.uniform(-5, 5, 20))
    S = S.astype(np.float32)
    shift, scale = oracle.fp8_calibrate(S)
    mn, mx = S.min(0).astype(np.float64), S.max(0).astype(np.float64)
    r = np.max(np.maximum(mx - shift, shift - mn))
    assert math.log2(scale) == int(math.log2(scale))
    assert scale * r <= 448.0 < 2.0 * scale * r
    codes = oracle.fp8_encode(S, shift, scale)
    assert codes.dtype == np.uint8 and not np.any((codes & 0x7F) == 0x7F)
    y = (S - shift) * np.float32(scale)
    back = oracle.to_f32(codes).astype(np.float64)
    # E4M3 keeps 3 mantissa bits: relative error at most 2^-4 (or 2^-10 absolute)
    assert np.all(np.abs(back - y) <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-12)
    dec = oracle.fp8_decode(back.astype(np.float32), shift, scale).astype(np.float64)
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) / scale
    assert np.all(np.abs(dec - S) <= bound + 1e-6 * (np.abs(S) + np.abs(shift)))
    edge = np.array([[-448.0 / 64], [448.0 / 64]], np.float32)
    assert oracle.fp8_calibrate(edge)[1] == 64.0
    assert oracle.fp8_calibrate(np.full((3, 2), 5.0, np.float32))[1] == 1.0
    far = np.full((1, 20), 1e9, np.float32)
    assert np.all(oracle.fp8_encode(far, shift, scale) == 0x7E)
    assert np.all(oracle.fp8_encode(-far, shift, scale) == 0xFE)


def test_fp8_training_closing_mean_is_exact_mean_of_codes():
    S = datagen.tiny(n=5000, d=16, seed=9)
    shift, scale = oracle.fp8_calibrate(S)
    X = oracle.fp8_encode(S, shift, scale)
    res = oracle.train(X, 40, 2.0, seed=5)
    Xv = oracle.to_f32(X).astype(np.float64)
    for j in range(40):
        m = res.labels == j
        if m.any():
            np.testing.assert_allclose(res.centroids[j], Xv[m].mean(axis=0), rtol=1e-6, atol=1e-6)
    # the search uses the centroids rounded to E4M3: x = 1 against 0.95 and
    # 1.06: as values 0.95 is nearer, but they round to 0.9375 and 1.0
    x1 = oracle.e4m3_bits(np.array([[1.0]], np.float32))
    c2 = np.array([[0.95], [1.06]], np.float32)
    assert oracle.e4m3_round(c2).ravel().tolist() == [0.9375, 1.0]
    assert oracle.assign(x1, oracle.search_centroids(c2, x1))[0].tolist() == [1]
    assert oracle.assign(x1, c2)[0].tolist() == [0]


def test_int8_training_closing_mean_is_exact_mean_of_codes():
    """Training on int8 codes: the centroids live in code space (fp32), the
    search uses their int8 rounding, and the closing mean is the exact mean of
    the codes the last pass assigned."""
    S = datagen.tiny(n=6000, d=16, seed=9)
    shift, scale = oracle.int8_calibrate(S)
    X = oracle.int8_encode(S, shift, scale)
    res = oracle.train(X, 48, 2.0, seed=5)
    lab = res.labels
    assert np.all(lab >= 0)
    for j in range(48):
        m = lab == j
        if m.any():
            np.testing.assert_allclose(res.centroids[j], X[m].astype(np.float64).mean(axis=0),
                                       rtol=0, atol=1e-4)
    # the search of int8 data uses the rounded centroids: x = 1 against 0.3 and
    # 1.6 is nearer 1.6, but against their codes 0 and 2 it is a tie, won by 0
    x1 = np.array([[1]], np.int8)
    c2 = np.array([[0.3], [1.6]], np.float32)
    assert oracle.assign(x1, oracle.search_centroids(c2, x1))[0].tolist() == [0]
    assert oracle.assign(x1, c2)[0].tolist() == [1]


def test_fractional_last_pass_labels():
    X = datagen.tiny(n=2000, d=16, seed=3)
    res = oracle.train(X, 16, 1.5, seed=5, batch_size=256)
    visited = oracle.perm_range(2000, 5, oracle.STREAM_PERM, 1, 0, 1000)
    assert np.all(res.labels[visited] >= 0)
    mask = np.ones(2000, bool)
    mask[visited] = False
    assert np.all(res.labels[mask] == -1)


# ---------------------------------------------------------------------------
# revival
# ---------------------------------------------------------------------------

def test_revival_splits_a_live_cluster():
    """A cluster whose count is below a tenth of the mean is refilled by
    splitting a live one: both halves carry half the donor's count, and the
    two centroids sit symmetrically around the donor's."""
    rng = np.random.default_rng(8)
    X = rng.standard_normal((2000, 8)).astype(np.float32)
    X[:10] += 100.0  # a far clump: the centroid started there starves
    res = oracle.train(X, 8, 2.0, seed=3, batch_size=100)
    assert len(res.split_log) > 0
    for t, j, i in res.split_log:
        assert t % 5 == 4 and j != i
    res_off = oracle.train(X, 8, 2.0, seed=3, batch_size=100, unused_threshold=0)
    assert res_off.split_log == []


def test_revival_mechanics_single_split():
    k, d = 5, 6
    N = np.array([10.0, 0.5, 20.0, 30.0, 40.0], dtype=np.float32)
    S = (np.arange(k * d, dtype=np.float32).reshape(k, d) + 1) * N[:, None]
    C = S / N[:, None]
    log = []
    oracle._revive(9, 1234, 0.1, N, S, C, log)
    assert len(log) == 1
    t, j, i = log[0]
    assert (t, j) == (9, 1) and i != 1
    assert N[j] == N[i]
    sig = oracle.split_signs(1234, 9, 1, d)
    base = (np.arange(d, dtype=np.float32) + 1 + i * d)
    np.testing.assert_allclose(C[j], base * (1 + 2**-10 * sig), rtol=1e-6)
    np.testing.assert_allclose(C[i], base * (1 - 2**-10 * sig), rtol=1e-6)


def test_revival_donor_frequency_is_size_proportional():
    """Over many independent checks, donors are picked in proportion to N."""
    Nlive = np.array([1.0, 2.0, 3.0, 4.0], dtype=np.float32)
    picks = np.zeros(4)
    for t in range(4000):
        N = np.concatenate([Nlive, np.zeros(1, np.float32)])
        S = np.ones((5, 2), np.float32) * N[:, None]
        C = np.ones((5, 2), np.float32)
        log = []
        oracle._revive(t, 77, 0.1, N, S, C, log)
        picks[log[0][2]] += 1
    freq = picks / picks.sum()
    np.testing.assert_allclose(freq, Nlive / Nlive.sum(), atol=0.025)


def test_revival_reduces_dead_clusters():
    """The trend of the blog's revival ablation (third change, the table for
    DEEP at k = 16,384 over 5 passes: a few dozen dead clusters with revival
    against thousands without, and a lower test loss with it), at a
    deep-like shape with the same rows per cluster (n / k = 64, 5 passes):
    without revival a few percent of the clusters end under the threshold,
    with it at least ten times fewer, and the loss is lower."""
    k = 1024
    X = datagen.deep(n=65536, d=96, seed=3)
    on = oracle.train(X, k, 5.0, seed=1)
    off = oracle.train(X, k, 5.0, seed=1, unused_threshold=0.0)
    assert off.split_log == []
    th_off = 0.1 * float(np.sum(off.N.astype(np.float64))) / k
    dead_off = int(np.sum(off.N.astype(np.float64) < th_off))
    assert dead_off >= 16, dead_off
    assert 10 * on.dead_at_end <= dead_off, (on.dead_at_end, dead_off)
    assert len(on.split_log) >= dead_off
    assert oracle.mse(X, on.centroids) < oracle.mse(X, off.centroids)


# Slow EMA (blog, section on what e-means changes: a second, slower EMA for
# unseen data; its decay is a reading: beta_t = alpha_t / kappa over the last pass)

def test_slow_ema_kappa_one_is_the_ema():
    """kappa = 1 makes the slow pair the running pair itself: the slow
    centroids equal the EMA centroids bit for bit, revivals in the last pass
    included."""
    X = datagen.tiny(n=3000, d=16, seed=9)
    res = oracle.train(X, 100, 2.0, seed=5, slow_ema=1.0)
    last0 = sum(res.recipe["steps_per_pass"][:-1])
    assert any(t >= last0 for t, _, _ in res.split_log), "no revival in the last pass"
    assert np.array_equal(res.slow_centroids, res.ema_centroids)
    assert np.array_equal(res.slow_N, res.N)
    with pytest.raises(ValueError):
        oracle.train(X, 32, 2.0, seed=5, slow_ema=0.5)


def test_slow_ema_closed_form_one_cluster():
    """With one cluster every row of a step goes to it, so both averages are
    fixed weighted sums of the batch sums: the running pair weighs step t by
    a_t prod_{u>t} (1 - a_u) up to the last pass, and the slow pair carries
    that on with b_u = a_u / kappa through the last pass."""
    n, d, T, kappa, seed, B = 2000, 16, 3.0, 4.0, 7, 256
    X = datagen.tiny(n=n, d=d, seed=3)
    res = oracle.train(X, 1, T, seed=seed, slow_ema=kappa, batch_size=B, unused_threshold=0.0)
    rc = res.recipe
    al = res.alphas.astype(np.float64)
    steps, sums, cnt, in_last = [], [], [], []
    for e, rows_e in enumerate(rc["epoch_rows"]):
        for s in range(rc["steps_per_pass"][e]):
            Bt = min(B, rows_e - s * B)
            rows = oracle.perm_range(n, seed, oracle.STREAM_PERM, e, s * B, Bt)
            sums.append(X[rows].astype(np.float64).sum(axis=0))
            cnt.append(float(Bt))
            in_last.append(e == len(rc["epoch_rows"]) - 1)
    S_tot = len(cnt)
    t0 = in_last.index(True)
    beta = np.array([np.float64(np.float32(al[t] / kappa)) for t in range(S_tot)])
    w = np.zeros(S_tot)
    for t in range(S_tot):
        if t < t0:    # running pair up to the last pass, then the slow decay
            w[t] = al[t] * np.prod(1.0 - al[t + 1:t0]) * np.prod(1.0 - beta[t0:])
        else:
            w[t] = beta[t] * np.prod(1.0 - beta[t + 1:])
    N2 = float(np.dot(w, cnt))
    S2 = np.dot(w, np.array(sums))
    np.testing.assert_allclose(res.slow_N[0], N2, rtol=1e-5)
    np.testing.assert_allclose(res.slow_centroids[0], S2 / N2, rtol=1e-5, atol=1e-6)
    # and it differs from the EMA centroid (the slow pair forgets less)
    assert not np.allclose(res.slow_centroids[0], res.ema_centroids[0], rtol=1e-4, atol=1e-6)


# UINT8 data (README "Data precision": INT8 and UINT8 input numbers)

def test_u8_rounding_decode_and_brute_force():
    r = oracle.u8_round(np.array([0.5, 1.5, 2.5, 254.5, 255.4, 255.6, 300.0, -3.0, -0.4, 7.49],
                                 np.float32))
    assert r.tolist() == [0, 2, 2, 254, 255, 255, 255, 0, 0, 7]   # ties to even, clamped
    # the C side reads every byte as its unsigned value (distance to 0 = v^2)
    allb = np.arange(256, dtype=np.uint8).reshape(-1, 1).view(oracle.U8)
    _, d1, _ = oracle.assign(allb, np.zeros((1, 1), np.float32))
    assert np.array_equal(d1, np.arange(256, dtype=np.float64) ** 2)
    # exact integer argmin against a pure-Python loop (ties to the lowest index)
    rng = np.random.default_rng(4)
    raw = rng.integers(0, 256, size=(40, 5)).astype(np.uint8)
    Q = rng.integers(0, 256, size=(9, 5)).astype(np.float32)
    Q[3] = Q[7]                                              # a tied pair
    raw[0] = Q[3].astype(np.uint8)                           # exact hit on the pair
    lab, d1, _ = oracle.assign(raw.view(oracle.U8), Q)
    for i in range(len(raw)):
        dd = [sum((int(raw[i, t]) - int(Q[j, t])) ** 2 for t in range(5)) for j in range(len(Q))]
        assert lab[i] == dd.index(min(dd)) and d1[i] == min(dd)
    assert lab[0] == 3 and d1[0] == 0
    # the GPU's form of the same search: rows and codes shifted by -128 as int8
    s_lab, s_d1, _ = oracle.assign((raw.astype(np.int16) - 128).astype(np.int8), Q - 128)
    assert np.array_equal(s_lab, lab) and np.array_equal(s_d1, d1)


def test_u8_training_closing_mean_and_search():
    X = datagen.make("codes-u8", 6000, 24, seed=5)
    res = oracle.train(X, 48, 2.0, seed=3)
    Xv = X.view(np.uint8).astype(np.float64)
    for j in range(48):
        m = res.labels == j
        if m.any():
            np.testing.assert_allclose(res.centroids[j], Xv[m].mean(axis=0), rtol=1e-6)
    # the search uses the centroids rounded to uint8: x = 10 against 10.6 and
    # 9.45: as values the second is nearer, but they round to 11 and 9, a tie
    # that goes to the lower index
    x = np.array([[10]], np.uint8).view(oracle.U8)
    c2 = np.array([[10.6], [9.45]], np.float32)
    assert oracle.assign(x, c2)[0].tolist() == [1]
    assert oracle.assign(x, oracle.search_centroids(c2, x))[0].tolist() == [0]


# On-the-fly converters of fp32 data (README "Data precision", fp32 rows
# converted batch by batch; centering)

def test_converter_centering_is_the_search_of_the_offset_free_data():
    """Centering subtracts the shift before rounding: data 1000 + y with y
    and the shift exact in fp32 is searched exactly as y itself, while the
    plain bf16 cast of 1000 + y loses y's low digits."""
    rng = np.random.default_rng(8)
    Y = (rng.integers(-512, 512, size=(600, 12)) / 256.0).astype(np.float32)
    CY = (rng.integers(-512, 512, size=(40, 12)) / 256.0).astype(np.float32)
    shift = np.full(12, 1000.0, np.float32)
    X, C = Y + shift, CY + shift                  # exact in fp32
    cen = oracle.Converter("bf16", shift)
    lab, d1, _ = oracle.assign(cen.rows(X), cen.centroids(C))
    ref, r1, _ = oracle.assign(oracle.bf16_bits(Y), oracle.bf16_round(CY))
    assert np.array_equal(lab, ref) and np.array_equal(d1, r1)
    plain = oracle.Converter("bf16")
    lab2, _, _ = oracle.assign(plain.rows(X), plain.centroids(C))
    assert not np.array_equal(lab2, ref)          # the offset costs the cast its digits
    # fp16 centering, same identity
    c16 = oracle.Converter("f16", shift)
    lab3, e1, _ = oracle.assign(c16.rows(X), c16.centroids(C))
    ref3, s1, _ = oracle.assign(Y.astype(np.float16), oracle.f16_round(CY))
    assert np.array_equal(lab3, ref3) and np.array_equal(e1, s1)


def test_fp8_converter_on_grid_data_is_exact():
    """Data and centroids on the FP8 converter's grid (shift + E4M3 value /
    scale, exact in fp32 for a shift in quarters) convert without loss: the
    rows become the codes, and the search in code units finds the exact fp32
    labels, its distances divided by scale^2 equal to the data-space ones."""
    codes = datagen.codes_e4m3(3000, 16, m=32, seed=13)
    shift = (np.arange(16, dtype=np.float32) - 8.0) / 4.0
    scale = 64.0
    X = (shift + oracle.to_f32(codes) / np.float32(scale)).astype(np.float32)
    conv = oracle.Converter("f8", shift, scale)
    assert np.array_equal(conv.rows(X), codes)
    C = X[np.random.default_rng(3).choice(len(X), 40, replace=False)].copy()
    assert np.array_equal(conv.centroids(C), conv.unrounded(C))     # on the grid
    lab, d1, _ = oracle.assign(conv.rows(X), conv.centroids(C))
    ref, r1, _ = oracle.assign(X, C)
    assert np.array_equal(lab, ref)
    assert np.array_equal(d1 / scale ** 2, r1)
    # training with the converter reports its error in data units: one Lloyd-
    # like step (B = n, alpha = 1) from the same rows matches the fp32 search
    a = oracle.train(X, 24, 1.0, seed=4, batch_size=len(X), alpha0=1.0, unused_threshold=0.0,
                     search="f8", search_shift=shift, search_scale=scale)
    b = oracle.train(X, 24, 1.0, seed=4, batch_size=len(X), alpha0=1.0, unused_threshold=0.0)
    assert np.array_equal(a.labels, b.labels)
    np.testing.assert_allclose(a.obj, b.obj, rtol=1e-12)
    # the alias: bf16_search is the plain bf16 converter
    Z = datagen.tiny(n=2000, d=8, seed=2)
    r1 = oracle.train(Z, 16, 2.0, seed=1, bf16_search=True)
    r2 = oracle.train(Z, 16, 2.0, seed=1, search="bf16")
    assert np.array_equal(r1.labels, r2.labels) and np.array_equal(r1.centroids, r2.centroids)


# ---------------------------------------------------------------------------
# Lloyd's empty-cluster split (Faiss's k-means splits a cluster left without
# rows off a large one; reading R9)


def test_lloyd_without_empty_clusters_is_plain_lloyd():
    """When no cluster is ever left without rows the split never fires: the
    result equals plain Lloyd, which a brute-force loop over scipy's cdist
    reproduces (nearest centroid, lowest index on ties, exact means)."""
    X = datagen.tiny(n=4000, d=16, seed=5)
    k, iters = 64, 6
    log = []
    C, hist = oracle.lloyd(X, k, iters, seed=3, split_log=log)
    Cp, hp = oracle.lloyd(X, k, iters, seed=3, split_empty=False)
    assert log == []
    assert np.array_equal(C, Cp) and hist == hp
    W = X[oracle.init_rows(len(X), k, 3)].astype(np.float64)
    for _ in range(iters):
        lab = np.argmin(cdist(X.astype(np.float64), W, "sqeuclidean"), axis=1)
        assert np.bincount(lab, minlength=k).min() > 0
        for j in range(k):
            W[j] = X[lab == j].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(C, W, rtol=0, atol=2e-6)


def test_lloyd_splits_every_empty_cluster_off_the_live_ones():
    """Six copies of one row and k = 3: every starting centroid is that row,
    the first takes all six rows (lowest index on ties) and the other two are
    empty. Both are refilled from the only live cluster, one after the other
    in index order, so the donor's half is halved again; the second iteration
    then gives all rows to the nearest of the three split centroids and that
    one returns to the row itself. The last iteration is not split."""
    a = np.array([3.0, -1.5, 0.25, 8.0, 2.0], dtype=np.float32)
    X = np.tile(a, (6, 1))
    d = len(a)
    log = []
    C, hist = oracle.lloyd(X, 3, 2, seed=7, split_log=log)
    assert [(t, j) for t, j, _ in log] == [(0, 1), (0, 2)]
    assert [i for _, _, i in log] == [0, 0]
    e = 2.0 ** -10
    s1 = oracle.split_signs(7, 0, 1, d).astype(np.float64)
    s2 = oracle.split_signs(7, 0, 2, d).astype(np.float64)
    a64 = a.astype(np.float64)
    after = np.stack([a64 * (1 - e * s1) * (1 - e * s2), a64 * (1 + e * s1),
                      a64 * (1 - e * s1) * (1 + e * s2)])
    win = int(np.argmin(((after - a64) ** 2).sum(axis=1)))
    want = after.copy()
    want[win] = a64
    np.testing.assert_allclose(C, want, rtol=1e-6, atol=0)
    assert hist[0] == 0.0 and hist[1] > 0.0


def test_lloyd_split_keeps_the_donor_mean_and_lowers_the_loss():
    """On the embedding-like mixture (Zipf weights) plain Lloyd leaves
    clusters empty; here every row also appears twice, so that starting
    centroids drawn from both copies of a row leave the second one empty from
    the first iteration on. The clusters split after the first iteration are
    exactly those the brute-force assignment (scipy's cdist, lowest index on
    ties) leaves without rows, in index order, each refilled from a cluster
    that has rows; a donor split once sits with its new cluster symmetrically
    about its mean, (c_i + c_j) / 2 = mean_i; and with the splits the loss
    ends lower."""
    X0 = datagen.make("embedding", 6_000, 768, seed=23)
    X = np.concatenate([X0, X0])
    k = 256
    W = X[oracle.init_rows(len(X), k, 1234)].astype(np.float64)
    lab0 = np.argmin(cdist(X.astype(np.float64), W, "sqeuclidean"), axis=1).astype(np.int32)
    cnt = np.bincount(lab0, minlength=k)
    seen = {}
    log = []
    oracle.lloyd(X, k, 2, 1234, split_log=log,
                 labels_for_step=lambda i, _: lab0 if i == 0 else np.zeros(len(X), np.int32),
                 check_hook=lambda chk: seen.__setitem__(chk["t"], chk["C32"].copy()))
    assert all(t == 0 for t, _, _ in log)
    assert [j for _, j, _ in log] == list(np.nonzero(cnt == 0)[0]) and len(log) > 0
    donors = [i for _, _, i in log]
    assert all(cnt[i] > 0 for i in donors)
    Cs = seen[1].astype(np.float64)  # the centroids the second iteration searched
    checked = 0
    for _, j, i in log:
        if donors.count(i) == 1:
            mean_i = X[lab0 == i].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose((Cs[i] + Cs[j]) / 2, mean_i, rtol=0, atol=1e-6)
            checked += 1
    assert checked > 0
    iters = 4
    C, _ = oracle.lloyd(X, k, iters, 1234)
    Cp, _ = oracle.lloyd(X, k, iters, 1234, split_empty=False)
    assert oracle.mse(X, C) < oracle.mse(X, Cp)
