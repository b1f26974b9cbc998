"""fp32 data converted on the fly for the search (README "Data precision",
the column for fp32 rows converted batch by batch): the bf16 and fp16 casts, with and without
centering, and the calibrated FP8 converter, against the oracle's Converter.
Labels are checked within the band of the search format, distances in data
units (the converted-unit distance divided by scale^2)."""
import numpy as np
import pytest

import oracle
from mini_means_amd import datagen

from parity import check_dists, check_labels, lockstep, obj_atol, rel_l2, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mini_means_amd
    mini_means_amd.lib()
    return mini_means_amd


def _centroids(X, k, seed):
    rng = np.random.default_rng(seed)
    C = X[rng.choice(len(X), size=k, replace=len(X) < k)].astype(np.float32)
    C += np.float32(0.05) * rng.standard_normal(C.shape).astype(np.float32) \
        * np.float32(np.abs(X).mean() + 1e-3)
    return np.ascontiguousarray(C)


def _setup(mm, X, fmt, center):
    """(GPU options, oracle Converter) for a format; center: the column mean
    of the first 4096 rows (casts) or, for f8, the calibrated shift."""
    import torch
    if fmt == "f8":
        shift, scale = mm.fp8_calibrate(torch.from_numpy(X[:4096]).cuda())
        sh = shift.cpu().numpy()
        return (dict(search="f8", search_shift=shift, search_scale=scale),
                oracle.Converter("f8", sh, scale))
    if center:
        sh = X[:4096].astype(np.float64).mean(axis=0).astype(np.float32)
        return (dict(search=fmt, search_shift=torch.from_numpy(sh).cuda()),
                oracle.Converter(fmt, sh))
    return dict(search=fmt), oracle.Converter(fmt)


ASSIGN = [("embedding", 2000, 768, 300, "f16", False), ("sift", 1500, 128, 257, "f16", True),
          ("sift", 1000, 128, 129, "bf16", True), ("deep", 3000, 96, 1000, "bf16", False),
          ("embedding", 1000, 768, 257, "f8", False), ("tiny", 777, 37, 50, "f8", False),
          ("tiny", 500, 40, 20, "f16", True), ("sift", 900, 64, 300, "f8", False)]


@pytest.mark.parametrize("gen,n,d,k,fmt,center", ASSIGN)
def test_assign_with_converter(mm, gen, n, d, k, fmt, center):
    import torch
    X = datagen.make(gen, n, d, seed=43)
    C = _centroids(X, k, 17)
    kw, conv = _setup(mm, X, fmt, center)
    lab, dist = mm.assign(to_device(X), torch.from_numpy(C).cuda(), **kw)
    lab, dist = lab.cpu().numpy(), dist.cpu().numpy()
    Xs, Cs = conv.rows(X), conv.centroids(C)
    olab, d1, d2 = oracle.assign(Xs, Cs)
    what = f"{fmt}{'-centered' if center else ''} {gen} {n}x{d} k={k}"
    check_labels(Xs, Cs, None, lab, olab, d1, d2, what=what)
    check_dists(Xs, Cs, None, lab, dist * np.float32(conv.scale2), what=what)


def test_centering_keeps_the_digits_far_from_the_origin(mm):
    """README "Data precision", centering: vectors far from the origin lose
    their differences to a plain 16-bit cast; with centering the search sees
    them again (assignment error against the exact fp32 labels)."""
    import torch
    rng = np.random.default_rng(5)
    Y = rng.standard_normal((3000, 32)).astype(np.float32)
    X = (Y + np.float32(3000.0)).astype(np.float32)
    # centroids near data rows at the data's own spread (fp16 spacing at 3000 is 2)
    C = (X[rng.choice(len(X), 64, replace=False)]
         + np.float32(0.3) * rng.standard_normal((64, 32)).astype(np.float32))
    exact, _, _ = oracle.assign(X, C)
    plain, _ = mm.assign(to_device(X), torch.from_numpy(C).cuda(), search="f16")
    sh = torch.full((32,), 3000.0, device="cuda")
    cent, _ = mm.assign(to_device(X), torch.from_numpy(C).cuda(), search="f16", search_shift=sh)
    miss_plain = np.mean(plain.cpu().numpy() != exact)
    miss_cent = np.mean(cent.cpu().numpy() != exact)
    assert miss_cent < 0.01 < miss_plain, (miss_cent, miss_plain)


TRAIN = [("emb-f16", "embedding", 12_000, 768, 256, 2.0, "f16", False, {}),
         ("sift-bf16c", "sift", 20_000, 128, 1024, 2.0, "bf16", True, {}),
         ("sift-f16c", "sift", 20_000, 128, 1024, 2.0, "f16", True, {}),
         ("emb-f8", "embedding", 12_000, 768, 256, 2.0, "f8", False, {}),
         ("ragged-f8", "tiny", 5_003, 37, 77, 1.5, "f8", False, dict(batch_size=700)),
         ("deep-f16-sph", "deep", 30_000, 96, 1024, 2.0, "f16", False, dict(spherical=True))]


@pytest.mark.parametrize("name,gen,n,d,k,T,fmt,center,o", TRAIN, ids=[c[0] for c in TRAIN])
def test_train_with_converter_lockstep(mm, name, gen, n, d, k, T, fmt, center, o):
    import torch
    seed = 1234
    X = datagen.make(gen, n, d, seed=21)
    kw, conv = _setup(mm, X, fmt, center)
    out = mm.train(to_device(X), k, T, seed, trace=True, counts=True, split_log_cap=1 << 16,
                   **kw, **o)
    torch.cuda.synchronize()
    res, summ = lockstep(X, out, k, T, seed, search=conv.fmt, search_shift=conv.shift,
                         search_scale=conv.scale, **o)
    assert summ["steps"] == res.recipe["total_steps"]
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert out.split_log == [tuple(s) for s in res.split_log]
    assert rel_l2(out.centroids.cpu().numpy(), res.centroids) <= 1e-4
    atol = obj_atol(conv.rows(X)) / conv.scale2
    np.testing.assert_allclose(out.stats["obj"], res.obj, rtol=1e-4, atol=atol)


def test_stream_with_converter(mm):
    """The streaming calls with the FP8 converter, batches fed in two pieces,
    in lockstep with the oracle."""
    from test_gpu_stream import _stream_run
    n, d, k, T, seed = 8_000, 64, 128, 2.0, 99
    X = datagen.make("embedding", n, d, seed=7)
    kw, conv = _setup(mm, X, "f8", False)
    out = _stream_run(mm, X, k, T, seed, pieces=2, **kw)
    res, _ = lockstep(X, out, k, T, seed, search="f8", search_shift=conv.shift,
                      search_scale=conv.scale)
    assert np.array_equal(out.counts.cpu().numpy(), res.N)
    assert rel_l2(out.centroids.cpu().numpy(), res.centroids) <= 1e-4
    np.testing.assert_allclose(out.stats["obj"], res.obj, rtol=1e-4,
                               atol=obj_atol(conv.rows(X)) / conv.scale2)


def test_converter_rules(mm):
    import torch
    X = to_device(datagen.make("tiny", 100, 8, seed=1))
    C = X[:4].contiguous()
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        mm.assign(X.half(), C, search="f16")                        # fp32 data only
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        mm.assign(X, C, search="f8")                                # no shift / scale
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        mm.assign(X, C, search="f8", search_shift=torch.zeros(8, device="cuda"),
                  search_scale=3.0)                                 # not a power of two
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        mm.train(X, 4, 1.0, spherical=True, search="bf16",
                 search_shift=torch.zeros(8, device="cuda"))        # no centering in spherical
