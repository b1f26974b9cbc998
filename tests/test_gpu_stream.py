"""Streaming training (README "Data too big for memory") on the GPU against the
oracle: the caller feeds the batches (here in the order of the library's own
sampler, so that the oracle can replay the run), and the oracle checks every
label in lockstep as for emeans_train."""
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from mini_means_amd import datagen

from parity import LOW_PRECISION, check_labels, lockstep, obj_atol, rel_l2, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mini_means_amd
    mini_means_amd.lib()
    return mini_means_amd


def _start(Xd, n, k, seed):
    """The starting rows emeans_train would take (first k of the init permutation)."""
    import torch
    idx = torch.from_numpy(oracle.init_rows(n, k, seed).astype(np.int64)).to(Xd.device)
    return Xd[idx].float().contiguous()


def _stream_run(mm, X, k, T, seed, pieces=1, keep=False, **kw):
    """Feed every batch of the schedule (rows from emeans_batch_rows), each as
    `pieces` accumulate calls followed by one update. With keep, the model
    stays open (out.model) after finalize."""
    import torch
    Xd = to_device(X)
    n = X.shape[0]
    em = mm.begin(n, _start(Xd, n, k, seed), T, seed, dtype=Xd.dtype, counts=True,
                  split_log_cap=1 << 16, **kw)
    B = em.recipe["batch_size"]
    trace = []
    labels = torch.full((n,), -1, dtype=torch.int32, device=Xd.device)
    last = len(em.recipe["epoch_rows"]) - 1
    for e, rows_e in enumerate(em.recipe["epoch_rows"]):
        for s0 in range(0, rows_e, B):
            nb = min(B, rows_e - s0)
            rows = mm.batch_rows(n, seed, e, s0, nb).long()
            cuts = np.linspace(0, nb, pieces + 1).astype(int)
            labs = []
            for a, b in zip(cuts[:-1], cuts[1:]):
                if b > a:
                    labs.append(em.accumulate(Xd[rows[a:b]].contiguous()))
            em.update()
            lab = torch.cat(labs)
            trace.append(lab)
            if e == last:
                labels[rows] = lab
        em.end_epoch()
    C = em.finalize()
    torch.cuda.synchronize()
    out = SimpleNamespace(trace=torch.cat(trace), counts=em.counts, centroids=C, labels=labels,
                          stats=em.stats, split_log=em.split_log,
                          slow_centroids=em.slow_centroids, model=em if keep else None)
    if not keep:
        em.close()
    return out


STREAM = [
    ("tiny", "tiny", 10_000, 16, 64, 3.0, 1, {}),
    ("emb-small", "embedding", 12_000, 768, 256, 2.0, 1, {}),
    ("deep-pieces", "deep", 30_000, 96, 1024, 2.0, 3, {}),
    ("large-bf16", "large", 40_000, 128, 1024, 2.0, 2, {}),
    ("emb-small-sph", "embedding", 12_000, 768, 256, 2.0, 1, dict(spherical=True)),
    ("ragged-bf16s", "tiny", 5_003, 37, 77, 1.5, 2, dict(batch_size=700, bf16_search=True)),
    ("codes-pieces", "codes", 12_000, 64, 256, 2.0, 2, {}),
    ("f8-pieces", "codes8", 12_000, 64, 256, 2.0, 2, {}),
    ("f16-pieces", "deep-f16", 12_000, 96, 256, 2.0, 2, {}),
    ("slow-ema", "tiny", 3_000, 16, 100, 2.0, 2, dict(slow_ema=4.0)),
    ("u8-pieces", "codes-u8", 12_000, 64, 256, 2.0, 2, {}),
]


@pytest.mark.parametrize("name,gen,n,d,k,T,pieces,o", STREAM, ids=[c[0] for c in STREAM])
def test_stream_lockstep(mm, name, gen, n, d, k, T, pieces, o):
    seed = 1234
    X = datagen.make(gen, n, d, seed=21)
    out = _stream_run(mm, X, k, T, seed, pieces=pieces, **o)
    res, summ = lockstep(X, out, k, T, seed, **o)
    assert summ["steps"] == res.recipe["total_steps"]
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert out.split_log == [tuple(s) for s in res.split_log]
    assert np.array_equal(out.labels.cpu().numpy(), res.labels)
    tol = 1e-2 if X.dtype == np.uint16 else 1e-4
    assert rel_l2(out.centroids.cpu().numpy(), res.centroids) <= tol
    np.testing.assert_allclose(out.stats["obj"], res.obj, rtol=1e-4, atol=obj_atol(X))
    if o.get("slow_ema"):
        assert rel_l2(out.slow_centroids.cpu().numpy(), res.slow_centroids) <= tol


def test_stream_window_grouping_in_pieces(mm):
    """The window grouping adds each later piece of an update to the sums of
    the earlier ones: three pieces per 4096-row batch of narrow rows (a few
    rows per cluster on average), one cluster holding hundreds of rows."""
    n, d, k, T, seed, bs = 24_000, 64, 1024, 2.0, 1234, 4096
    X = datagen.make("tiny", n, d, seed=5)
    rng = np.random.default_rng(5)
    X[rng.choice(n, n // 4, replace=False)] = X[0]
    out = _stream_run(mm, X, k, T, seed, pieces=3, batch_size=bs)
    res, summ = lockstep(X, out, k, T, seed, batch_size=bs)
    assert summ["steps"] == res.recipe["total_steps"]
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert out.split_log == [tuple(s) for s in res.split_log]
    assert np.array_equal(out.labels.cpu().numpy(), res.labels)
    assert rel_l2(out.centroids.cpu().numpy(), res.centroids) <= 1e-4
    np.testing.assert_allclose(out.stats["obj"], res.obj, rtol=1e-4, atol=obj_atol(X))


def test_stream_rejects_rule_breaks(mm):
    """README "Data too big for memory" rules: batches of exactly the recipe's
    size except the last of a pass, every pass visits its rows, begin before
    and nothing after the last pass."""
    import torch
    X = datagen.make("tiny", 2000, 16, seed=3)
    Xd = to_device(X)
    em = mm.begin(2000, Xd[:20].contiguous(), 1.0, 7, batch_size=512)
    assert em.recipe["epoch_rows"] == [2000]
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        em.accumulate(Xd[:513].contiguous())           # larger than a batch
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        em.update()                                    # nothing accumulated
    em.accumulate(Xd[:300].contiguous())
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        em.update()                                    # 300 rows, not the last batch
    em.accumulate(Xd[300:512].contiguous())
    em.update()
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        em.end_epoch()                                 # 512 of 2000 rows
    for a in range(512, 2000, 512):
        em.accumulate(Xd[a:min(a + 512, 2000)].contiguous())
        em.update()
    em.end_epoch()
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        em.accumulate(Xd[:10].contiguous())            # all passes ended
    C = em.finalize()
    assert C.shape == (20, 16) and torch.isfinite(C).all()
    em.close()
    with pytest.raises(mm.EmeansError):
        em.update()


def test_train_from_host_lockstep(mm):
    """Host-resident data streamed through pinned buffers on a second stream.
    By default it starts from emeans_train's rows and visits the rows in the
    library sampler's order, so the oracle replays it with the plain recipe:
    lockstep parity as for emeans_train."""
    seed = 1234
    X = datagen.make("deep", 20_000, 96, seed=21)
    k, T = 512, 2.0
    import torch
    first = mm.batch_rows(len(X), seed, -1, 0, k).cpu().numpy()
    assert np.array_equal(first, oracle.init_rows(len(X), k, seed))
    res_h = mm.train_from_host(X, k, T, seed, trace=True, counts=True, split_log_cap=1 << 16)
    em = res_h.stream
    out = SimpleNamespace(trace=torch.from_numpy(res_h.trace), counts=em.counts,
                          centroids=res_h.centroids, stats=em.stats, split_log=em.split_log)
    res, summ = lockstep(X, out, k, T, seed)
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert out.split_log == [tuple(s) for s in res.split_log]
    assert np.array_equal(res_h.labels, res.labels)
    assert rel_l2(out.centroids.cpu().numpy(), res.centroids) <= 1e-4
    em.close()


CLOSING = [
    ("tiny", "tiny", 10_000, 16, 64, 2.0, {}),
    ("emb-frac", "embedding", 12_000, 768, 256, 1.5, {}),
    ("deep-sph", "deep", 30_000, 96, 1024, 2.0, dict(spherical=True)),
    ("large-bf16", "large", 40_000, 128, 1024, 2.0, {}),
    ("codes", "codes", 12_000, 64, 256, 2.0, {}),
    ("f16-search", "deep", 20_000, 96, 512, 2.0, dict(search="f16")),
]


@pytest.mark.parametrize("name,gen,n,d,k,T,o", CLOSING, ids=[c[0] for c in CLOSING])
def test_stream_final_closing_mean(mm, name, gen, n, d, k, T, o):
    """README "Several GPUs", final_closing_mean, after a streamed run that
    the oracle replays in lockstep:
    * replaying the rows in row order (blocks of 3000, not the batch cut) with
      the labels saved in the last pass (-1 for the rows a fractional pass
      skipped) gives the run's own closing mean;
    * replaying them without labels searches the final EMA centroids: every
      label is checked against the oracle's fp64 search of the oracle's EMA
      centroids (the tie band), and the centroids against the oracle's
      closing mean over the labels used."""
    import torch
    seed = 1234
    X = datagen.make(gen, n, d, seed=21)
    run = _stream_run(mm, X, k, T, seed, keep=True, **o)
    em = run.model
    res, _ = lockstep(X, run, k, T, seed, **o)
    tol = 1e-2 if X.dtype == np.uint16 else 1e-4
    assert rel_l2(run.centroids.cpu().numpy(), res.centroids) <= tol
    Xd = to_device(X)
    blocks = [Xd[a:a + 3000] for a in range(0, n, 3000)]
    saved = run.labels.cpu().numpy()
    if T % 1:
        assert np.sum(saved < 0) == n - int((T % 1) * n)
    used = em.final_closing_mean(blocks, saved.astype(np.int64), labels_out=True)
    assert np.array_equal(used.cpu().numpy(), saved)
    C1 = em.finalize().cpu().numpy()
    assert rel_l2(C1, res.centroids) <= tol
    assert rel_l2(C1, run.centroids.cpu().numpy()) <= 1e-5

    used = em.final_closing_mean(blocks, labels_out=True).cpu().numpy()
    C2 = em.finalize().cpu().numpy()
    sph = bool(o.get("spherical"))
    conv = oracle.converter(search=o.get("search"))
    Xs = conv.rows(X) if conv is not None else X
    Cs = conv.centroids(res.ema_centroids) if conv is not None else \
        oracle.search_centroids(res.ema_centroids, X)
    if sph:
        olab, s1, s2 = oracle.assign_ip(Xs, Cs)
        d1, d2, gd = -2.0 * s1, -2.0 * s2, -2.0 * oracle.dot_to(Xs, Cs, used)
    else:
        olab, d1, d2 = oracle.assign(Xs, Cs)
        gd = oracle.dist_to(Xs, Cs, used)
    C32 = conv.unrounded(res.ema_centroids) if conv is not None else res.ema_centroids
    check_labels(Xs, Cs, None, used, olab, d1, d2, gd, what=f"{name} replay",
                 C32=C32 if Xs.dtype in LOW_PRECISION else None, dot=sph)
    want, _ = oracle.final_closing_mean([X], res.ema_centroids, used, spherical=sph)
    assert rel_l2(C2, want) <= tol
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        em.final_closing_mean(blocks[:1], np.full(5, -1))      # fewer rows than labels
    em.close()


def test_stream_closing_replay_rules(mm):
    """The replay starts only after the last pass; labels outside [-1, k)
    are left out and reported by finalize."""
    import torch
    X = datagen.make("tiny", 2000, 16, seed=3)
    Xd = to_device(X)
    em = mm.begin(2000, Xd[:20].contiguous(), 1.0, 7, batch_size=512)
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        em.final_closing_mean([Xd[:100]])                      # the pass is still open
    for a in range(0, 2000, 512):
        em.accumulate(Xd[a:a + 512].contiguous())
        em.update()
    em.end_epoch()
    bad = np.zeros(2000, dtype=np.int32)
    bad[7] = 20                                                 # k = 20: out of range
    em.final_closing_mean([Xd], bad)
    with pytest.raises(mm.EmeansError, match="outside"):
        em.finalize()
    em.final_closing_mean([Xd], np.zeros(2000, dtype=np.int32))
    C = em.finalize().cpu().numpy()
    np.testing.assert_allclose(C[0], X.astype(np.float64).mean(0), rtol=0, atol=1e-5)
    em.close()
