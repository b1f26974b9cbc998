"""emeans_train on the GPU against the oracle.

Lockstep: the oracle replays the GPU run step by step, checks every label the
GPU produced against its own fp64 assignment on its own centroids, adopts
them, and the two states are then compared (running counts bit for bit, the
split log exactly, centroids to 1e-4 relative L2, final MSE to 1e-3).
Free run: the two run independently from the same seed.
"""
import numpy as np
import pytest

import oracle
from mini_means_amd import datagen

from parity import LOW_PRECISION, lockstep, obj_atol, rel_l2, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mini_means_amd
    mini_means_amd.lib()
    return mini_means_amd


def _gpu_train(mm, X, k, T, seed, **o):
    """mm.train with oracle-style options (unused_threshold: -1 default, 0 off)."""
    import torch
    ut = o.pop("unused_threshold", -1.0)
    out = mm.train(to_device(X), k, T, seed, unused_threshold=None if ut < 0 else ut,
                   trace=True, counts=True, split_log_cap=1 << 16, **o)
    torch.cuda.synchronize()
    return out


# (name, generator, n, d, k, T, extra options)
LOCKSTEP = [
    ("tiny", "tiny", 10_000, 16, 64, 5.0, {}),
    ("emb-small", "embedding", 12_000, 768, 256, 2.0, {}),
    ("deep-small", "deep", 30_000, 96, 1024, 3.0, {}),
    ("sift-small", "sift", 20_000, 128, 1024, 2.0, {}),
    ("large-small", "large", 40_000, 128, 1024, 2.0, {}),
    ("ragged", "tiny", 5_003, 37, 77, 1.5, dict(batch_size=700)),
    # narrow rows with Zipf-heavy clusters: spans holding a cluster of more
    # than 256 rows in a batch take the per-cluster grouping path plus overflow items
    ("zipf-narrow", "embedding", 20_000, 64, 64, 2.0, dict(batch_size=8192)),
    ("no-revival", "deep", 8_000, 96, 300, 2.0, dict(unused_threshold=0.0)),
    ("alpha1-lloyd", "tiny", 4_000, 16, 32, 1.0, dict(batch_size=4000, alpha0=1.0)),
    # fp32 data searched in bf16 (README "Data precision", the pages' GPU default)
    ("emb-small-bf16s", "embedding", 12_000, 768, 256, 2.0, dict(bf16_search=True)),
    ("deep-small-bf16s", "deep", 30_000, 96, 1024, 3.0, dict(bf16_search=True)),
    ("ragged-bf16s", "tiny", 5_003, 37, 77, 1.5, dict(batch_size=700, bf16_search=True)),
    # spherical e-means (README "Spherical e-means") on unit-norm data
    ("emb-small-sph", "embedding", 12_000, 768, 256, 2.0, dict(spherical=True)),
    ("deep-small-sph", "deep", 30_000, 96, 1024, 3.0, dict(spherical=True)),
    ("large-small-sph", "large", 40_000, 128, 1024, 2.0, dict(spherical=True)),
    # int8 codes (README "Data precision", INT8): exact integer search
    ("codes-small", "codes", 12_000, 768, 256, 2.0, {}),
    ("codes-ragged", "codes", 5_003, 37, 77, 1.5, dict(batch_size=700)),
    ("codes-deep", "codes", 30_000, 96, 1024, 3.0, {}),
    # FP8 E4M3 codes (README "Data precision", FP8)
    ("f8-small", "codes8", 12_000, 768, 256, 2.0, {}),
    ("f8-ragged", "codes8", 5_003, 37, 77, 1.5, dict(batch_size=700)),
    ("f8-deep", "codes8", 30_000, 96, 1024, 3.0, {}),
    # fp16 data (README "Data precision", FP16): fp16 search, fp32 sums
    ("f16-small", "embedding-f16", 12_000, 768, 256, 2.0, {}),
    ("f16-deep", "deep-f16", 30_000, 96, 1024, 3.0, {}),
    ("f16-ragged", "tiny-f16", 5_003, 37, 77, 1.5, dict(batch_size=700)),
    ("f16-sph", "embedding-f16", 12_000, 768, 256, 2.0, dict(spherical=True)),
    # uint8 data (README "Data precision", UINT8): exact integer search
    ("u8-small", "codes-u8", 12_000, 128, 256, 2.0, {}),
    ("u8-ragged", "codes-u8", 5_003, 37, 77, 1.5, dict(batch_size=700)),
    ("u8-sift", "sift-u8", 20_000, 128, 1024, 2.0, {}),
    # rows of 16-byte grouping units: 768 code bytes, 384 bf16 and fp16 values
    ("u8-wide", "codes-u8", 12_000, 768, 256, 2.0, {}),
    ("large-384", "large", 20_000, 384, 512, 2.0, {}),
    ("f16-384", "embedding-f16", 12_000, 384, 256, 2.0, {}),
]


@pytest.mark.parametrize("name,gen,n,d,k,T,o", LOCKSTEP, ids=[c[0] for c in LOCKSTEP])
def test_train_lockstep(mm, name, gen, n, d, k, T, o):
    seed = 1234
    X = datagen.make(gen, n, d, seed=21)
    out = _gpu_train(mm, X, k, T, seed, **dict(o))
    res, summ = lockstep(X, out, k, T, seed, **o)
    assert summ["steps"] == res.recipe["total_steps"]
    assert out.stats["batch_size"] == res.recipe["batch_size"]
    # running counts: same labels -> bit-identical fp32 recurrence
    assert np.array_equal(out.counts.cpu().numpy(), res.N), "running counts differ"
    # revivals: identical decisions
    assert out.split_log == [tuple(s) for s in res.split_log]
    assert out.stats["n_splits"] == len(res.split_log)
    assert out.stats["dead_at_end"] == res.dead_at_end
    # last-pass labels are the adopted trace
    assert np.array_equal(out.labels.cpu().numpy(), res.labels)
    tol = 1e-2 if X.dtype == np.uint16 else 1e-4
    C = out.centroids.cpu().numpy()
    err = rel_l2(C, res.centroids)
    assert err <= tol, f"centroids rel L2 {err:.3e}"
    m_gpu = oracle.mse(X, C)
    m_ref = oracle.mse(X, res.centroids)
    assert abs(m_gpu - m_ref) <= 1e-3 * m_ref
    np.testing.assert_allclose(out.stats["obj"], res.obj, rtol=1e-4, atol=obj_atol(X))
    if o.get("spherical"):
        nrm = np.linalg.norm(C.astype(np.float64), axis=1)
        assert np.all((np.abs(nrm - 1.0) < 1e-6) | (nrm == 0.0))


def _dup_heavy(n, d, frac, seed):
    """Seeded rows of the 64-centre mixture with a share `frac` of them replaced
    by one repeated row, so that one cluster holds hundreds of rows of every
    batch while the average cluster holds a few."""
    X = datagen.make("tiny", n, d, seed=seed)
    rng = np.random.default_rng(seed)
    X[rng.choice(n, int(frac * n), replace=False)] = X[0]
    return X


def test_train_lockstep_window_grouping_long_cluster(mm):
    """Narrow rows in batches of at most 8 rows per cluster on average are
    grouped by 8-slot windows of the bucketed order, each wave reading 64
    slots ahead; here one cluster holds about 700 rows of each 4096-row batch,
    so its wave finishes it in further 64-slot chunks."""
    X = _dup_heavy(24_000, 64, 0.25, 5)
    k, T, seed, bs = 1024, 2.0, 1234, 4096
    out = _gpu_train(mm, X, k, T, seed, batch_size=bs)
    trace = out.trace.cpu().numpy()
    assert bs <= 8 * k
    assert max(np.bincount(trace[s:s + bs], minlength=k).max()
               for s in range(0, len(trace), bs)) > 3 * 64
    res, summ = lockstep(X, out, k, T, seed, batch_size=bs)
    assert summ["steps"] == res.recipe["total_steps"]
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert out.split_log == [tuple(s) for s in res.split_log]
    assert np.array_equal(out.labels.cpu().numpy(), res.labels)
    assert rel_l2(out.centroids.cpu().numpy(), res.centroids) <= 1e-4
    np.testing.assert_allclose(out.stats["obj"], res.obj, rtol=1e-4, atol=obj_atol(X))


LLOYD = [("tiny", "tiny", 10_000, 16, 64, 8), ("emb-small", "embedding", 12_000, 768, 256, 4),
         ("large-small", "large", 40_000, 128, 1024, 3), ("codes", "codes", 12_000, 96, 200, 4),
         ("ragged", "tiny", 5_003, 37, 77, 5), ("f8", "codes8", 12_000, 128, 200, 4),
         ("f16", "sift-f16", 12_000, 128, 200, 4), ("u8", "codes-u8", 12_000, 64, 200, 4)]


@pytest.mark.parametrize("name,gen,n,d,k,iters", LLOYD, ids=[c[0] for c in LLOYD])
def test_lloyd_mode_lockstep(mm, name, gen, n, d, k, iters):
    """GPU Lloyd mode against the oracle's Lloyd, adopting the band-checked
    GPU labels every iteration: per-iteration MSE, the empty-cluster splits
    (identical decisions), final counts and centroids."""
    from parity import check_labels
    X = datagen.make(gen, n, d, seed=23)
    out = _gpu_train(mm, X, k, float(iters), 1234, lloyd=True)
    trace = out.trace.cpu().numpy().reshape(iters, n)
    last = {}

    def hook(chk):
        C32 = chk["C32"] if X.dtype in LOW_PRECISION else None
        check_labels(X, chk["C"], None, chk["given"], chk["oracle"], chk["d1"], chk["d2"],
                     chk["given_dist"], what=f"lloyd {name} iteration {chk['t']}", C32=C32)
        last["labels"] = chk["given"]

    splits = []
    C, hist = oracle.lloyd(X, k, iters, 1234, labels_for_step=lambda i, _: trace[i],
                           check_hook=hook, split_log=splits)
    np.testing.assert_allclose(out.stats["obj"], hist, rtol=1e-4, atol=obj_atol(X))
    counts = np.bincount(last["labels"], minlength=k).astype(np.float32)
    assert np.array_equal(out.counts.cpu().numpy(), counts)
    assert np.array_equal(out.labels.cpu().numpy(), last["labels"])
    tol = 1e-2 if X.dtype == np.uint16 else 1e-4
    err = rel_l2(out.centroids.cpu().numpy(), C)
    assert err <= tol, f"centroids rel L2 {err:.3e}"
    assert out.split_log == [tuple(v) for v in splits]
    assert out.stats["n_splits"] == len(splits)
    assert out.stats["dead_at_end"] == int(np.sum(counts == 0))
    if name == "emb-small":
        assert len(splits) > 10  # this case does leave clusters empty


# Revival draws at larger k, each with thousands of revivals: the speculated
# rounds up to k = 16384 (k6000, and k16384 with the full prefix tree), then
# 64 chunks of 64 V clusters, V = 8 just past it, V = 8 and 16 (live counts in
# global memory), and the generic path (k > 65536).
REVIVAL_K = [
    ("k6000", 24_000, 8, 6_000, 4_096),
    ("k16384", 50_000, 8, 16_384, 8_192),
    ("k16385", 50_000, 8, 16_385, 8_192),
    ("k20000", 60_000, 8, 20_000, 8_192),
    ("k40000", 100_000, 4, 40_000, 16_384),
    ("k66000", 140_000, 4, 66_000, 16_384),
]


@pytest.mark.parametrize("name,n,d,k,bs", REVIVAL_K, ids=[c[0] for c in REVIVAL_K])
def test_train_lockstep_revival_widths(mm, name, n, d, k, bs):
    seed = 1234
    X = datagen.make("tiny", n, d, seed=21)
    out = _gpu_train(mm, X, k, 2.0, seed, batch_size=bs)
    res, summ = lockstep(X, out, k, 2.0, seed, sample=256, rng_seed=2, batch_size=bs)
    assert len(res.split_log) > 100
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert out.split_log == [tuple(s) for s in res.split_log]
    assert np.array_equal(out.labels.cpu().numpy(), res.labels)
    assert rel_l2(out.centroids.cpu().numpy(), res.centroids) <= 1e-4


FREERUN = [
    ("tiny", "tiny", 10_000, 16, 64, 5.0),
    ("deep-small", "deep", 20_000, 96, 512, 3.0),
    ("emb-small", "embedding", 12_000, 768, 256, 2.0),
]


@pytest.mark.parametrize("name,gen,n,d,k,T", FREERUN, ids=[c[0] for c in FREERUN])
def test_train_free_run(mm, name, gen, n, d, k, T):
    """Independent runs from the same seed. While the two trajectories see the
    same labels they agree to the parity bar (centroids 1e-4, MSE 1e-3). A
    single near-tie label that the two sides legitimately resolve differently
    sends them onto different trajectories (the update is chaotic), so once
    the labels differ the final losses are compared with the oracle's own
    seed-to-seed spread instead."""
    seed = 1234
    X = datagen.make(gen, n, d, seed=22)
    Xh = datagen.make(gen, n // 2, d, seed=22, split=1)
    out = _gpu_train(mm, X, k, T, seed)
    res = oracle.train(X, k, T, seed)
    C = out.centroids.cpu().numpy()
    m_gpu, m_ref = oracle.mse(X, C), oracle.mse(X, res.centroids)
    h_gpu, h_ref = oracle.mse(Xh, C), oracle.mse(Xh, res.centroids)
    agree = np.mean(out.labels.cpu().numpy() == res.labels)
    if agree == 1.0:
        assert rel_l2(C, res.centroids) <= 1e-4
        assert abs(m_gpu - m_ref) <= 1e-3 * m_ref, (m_gpu, m_ref)
        assert abs(h_gpu - h_ref) <= 1e-3 * h_ref, (h_gpu, h_ref)
        return
    others = [oracle.train(X, k, T, s) for s in (seed + 1, seed + 2, seed + 3)]
    spread = np.std([oracle.mse(X, r.centroids) for r in [res] + others])
    hspread = np.std([oracle.mse(Xh, r.centroids) for r in [res] + others])
    assert abs(m_gpu - m_ref) <= max(1e-3 * m_ref, 3 * spread), (m_gpu, m_ref, spread)
    assert abs(h_gpu - h_ref) <= max(1e-3 * h_ref, 3 * hspread), (h_gpu, h_ref, hspread)


def test_train_finalisation_identity(mm):
    """Each returned centroid is the exact mean of the rows whose last-pass
    label it is (README: the closing mean costs nothing extra)."""
    X = datagen.deep(n=30_000, d=96, seed=5)
    out = _gpu_train(mm, X, 700, 2.0, 99)
    lab = out.labels.cpu().numpy()
    C = out.centroids.cpu().numpy()
    assert lab.min() >= 0
    cnt = np.bincount(lab, minlength=700)
    sums = np.zeros((700, 96))
    np.add.at(sums, lab, X.astype(np.float64))
    nz = cnt > 0
    means = sums[nz] / cnt[nz, None]
    assert rel_l2(C[nz], means) <= 1e-5


def test_train_every_row_once_per_pass(mm):
    X = datagen.tiny(n=3_000, d=16, seed=8)
    out = _gpu_train(mm, X, 20, 3.0, 5, batch_size=256)
    rc = oracle.recipe(3000, 16, 20, 3.0, batch_size=256)
    for e in range(3):
        rows = mm.batch_rows(3000, 5, e, 0, 3000).cpu().numpy()
        assert np.array_equal(np.sort(rows), np.arange(3000))
    assert out.trace.numel() == sum(rc["epoch_rows"])


def test_train_no_finalize_returns_ema(mm):
    X = datagen.tiny(n=4_000, d=16, seed=9)
    out = _gpu_train(mm, X, 32, 2.0, 3, finalize=False)
    res, _ = lockstep(X, out, 32, 2.0, 3, finalize=False)
    assert rel_l2(out.centroids.cpu().numpy(), res.ema_centroids) <= 1e-4


def test_train_k_equals_n_and_k1(mm):
    X = datagen.tiny(n=300, d=16, seed=4)
    out = _gpu_train(mm, X, 300, 1.0, 1, batch_size=300, alpha0=1.0, unused_threshold=0.0)
    # one Lloyd step from all rows as centroids: each row is its own centroid
    assert np.array_equal(np.sort(out.labels.cpu().numpy()), np.arange(300))
    out1 = _gpu_train(mm, X, 1, 2.0, 1)
    assert np.allclose(out1.centroids.cpu().numpy()[0], X.astype(np.float64).mean(0), atol=1e-5)


def test_train_repeatable(mm):
    """Two runs with the same seed visit the same batches. Within a cluster the
    fp32 summation order follows the atomic bucketing, so the runs may part
    at a near-tie; until then they agree to the parity bar."""
    X = datagen.deep(n=20_000, d=96, seed=6)
    a = _gpu_train(mm, X, 256, 2.0, 7)
    b = _gpu_train(mm, X, 256, 2.0, 7)
    la, lb = a.labels.cpu().numpy(), b.labels.cpu().numpy()
    Ca, Cb = a.centroids.cpu().numpy(), b.centroids.cpu().numpy()
    if np.array_equal(la, lb):
        assert rel_l2(Ca, Cb) <= 1e-4
    ma, mb = oracle.mse(X, Ca), oracle.mse(X, Cb)
    assert abs(ma - mb) <= 1e-2 * mb


def test_train_profile_per_pass_times(mm):
    """With profile set, each pass reports its device time; the passes cover the
    timed kernel classes, and a run cut short reports the passes it began."""
    X = datagen.deep(n=20_000, d=96, seed=8)
    out = _gpu_train(mm, X, 256, 2.5, 3, profile=True)
    st = out.stats
    assert st["n_passes"] == 3 and len(st["pass_ms"]) == 3
    assert all(v > 0.0 for v in st["pass_ms"])
    classes = sum(st[c] for c in ("ms_assign", "ms_bucket", "ms_group", "ms_update",
                                  "ms_revive", "ms_sample"))
    assert classes > 0.0
    assert classes <= 1.02 * sum(st["pass_ms"]) + 0.05
    assert sum(st["pass_ms"]) <= st["ms_total"] + 0.05
    cut = _gpu_train(mm, X, 256, 2.5, 3, profile=True, max_steps=1)
    assert cut.stats["pass_ms"][0] > 0.0 and cut.stats["pass_ms"][1:] == [0.0, 0.0]
    plain = _gpu_train(mm, X, 256, 2.5, 3)
    assert plain.stats["pass_ms"] == [0.0, 0.0, 0.0]


SLOW = [
    ("tiny-revive", "tiny", 3_000, 16, 100, 2.0, {}),
    ("emb-small", "embedding", 12_000, 768, 256, 2.0, {}),
    ("deep-sph", "deep", 30_000, 96, 1024, 2.5, dict(spherical=True)),
    ("large-bf16", "large", 40_000, 128, 1024, 2.0, {}),
    ("f16", "deep-f16", 12_000, 96, 256, 2.0, {}),
]


@pytest.mark.parametrize("name,gen,n,d,k,T,o", SLOW, ids=[c[0] for c in SLOW])
def test_train_slow_ema_lockstep(mm, name, gen, n, d, k, T, o):
    """The slow EMA (kappa = 4) against the oracle's on the adopted labels:
    the slow centroids to 1e-4 relative L2 (1e-2 for bf16 data, as the
    centroids), alongside the usual lockstep checks."""
    seed, kappa = 1234, 4.0
    X = datagen.make(gen, n, d, seed=21)
    out = _gpu_train(mm, X, k, T, seed, slow_ema=kappa, **dict(o))
    res, _ = lockstep(X, out, k, T, seed, slow_ema=kappa, **o)
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert out.split_log == [tuple(s) for s in res.split_log]
    tol = 1e-2 if X.dtype == np.uint16 else 1e-4
    SC = out.slow_centroids.cpu().numpy()
    err = rel_l2(SC, res.slow_centroids)
    assert err <= tol, f"slow centroids rel L2 {err:.3e}"
    assert rel_l2(out.centroids.cpu().numpy(), res.centroids) <= tol
    if o.get("spherical"):
        nrm = np.linalg.norm(SC.astype(np.float64), axis=1)
        assert np.all((np.abs(nrm - 1.0) < 1e-6) | (nrm == 0.0))


def test_train_slow_ema_kappa_one_and_early_stop(mm):
    """kappa = 1 runs the EMA's own recurrence: the slow centroids equal the
    EMA centroids of the same run bit for bit (revivals in the last pass
    included). A run stopped before its last pass returns the EMA centroids."""
    import torch
    X = to_device(datagen.make("tiny", 3_000, 16, seed=9))
    out = mm.train(X, 100, 2.0, 5, slow_ema=1.0, finalize=False, split_log_cap=4096)
    assert torch.equal(out.slow_centroids, out.centroids)
    last0 = sum(out.stats["steps_per_pass"][:-1])
    assert any(t >= last0 for t, _, _ in out.split_log)
    part = mm.train(X, 100, 2.0, 5, slow_ema=3.0, finalize=False, max_steps=3)
    assert torch.equal(part.slow_centroids, part.centroids)


def test_train_rejects_bad_args(mm):
    import torch
    X = torch.zeros((100, 8), device="cuda")
    with pytest.raises(mm.EmeansError):
        mm.train(X, 101)
    with pytest.raises(mm.EmeansError):
        mm.train(X, 10, T=0.0)
    with pytest.raises(mm.EmeansError):
        mm.train(X.double(), 10)
