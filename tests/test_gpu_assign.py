"""emeans_assign and emeans_batch_rows on the GPU against the oracle."""
import numpy as np
import pytest

import oracle
from mini_means_amd import datagen

from parity import check_dists, check_labels, to_device

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
    Xf = oracle.to_f32(X)
    idx = rng.choice(len(X), size=k, replace=len(X) < k)
    C = Xf[idx].astype(np.float32) + 0.05 * rng.standard_normal((k, X.shape[1])).astype(np.float32) \
        * np.float32(np.abs(Xf).mean() + 1e-3)
    return np.ascontiguousarray(C, dtype=np.float32)


def _run(mm, X, C):
    import torch
    Xd = to_device(X)
    Cd = torch.from_numpy(C).cuda()
    lab, dist = mm.assign(Xd, Cd)
    torch.cuda.synchronize()
    return lab.cpu().numpy(), dist.cpu().numpy()


CASES_F32 = [
    # (generator, n, d, k): several tiles, ragged tails in n, k and d
    ("tiny", 1000, 16, 64),
    ("tiny", 3001, 16, 130),
    ("embedding", 1000, 768, 257),
    ("embedding", 700, 100, 300),
    ("deep", 5000, 96, 1000),
    ("sift", 2000, 128, 513),
    ("tiny", 257, 5, 3),
    ("tiny", 130, 33, 200),
    ("tiny", 100, 1, 1),
    ("tiny", 129, 7, 129),
    ("sift", 300, 250, 17),
    ("embedding", 1500, 36, 700),
    ("embedding", 513, 1028, 520),
]


@pytest.mark.parametrize("gen,n,d,k", CASES_F32)
def test_assign_fp32(mm, gen, n, d, k):
    X = datagen.make(gen, n, d, seed=11)
    C = _centroids(X, k, 5)
    lab, dist = _run(mm, X, C)
    olab, d1, d2 = oracle.assign(X, C)
    check_labels(X, C, None, lab, olab, d1, d2, what=f"{gen} {n}x{d} k={k}")
    check_dists(X, C, None, lab, dist, what=f"{gen} {n}x{d} k={k}")


CASES_BF16 = [(2000, 128, 300), (1000, 64, 129), (777, 40, 50), (500, 37, 20), (300, 256, 1),
              (900, 520, 300), (600, 1024, 257), (4097, 768, 1025), (300, 768, 1)]


CASES_BF16_SEARCH = [("sift", 2000, 128, 300), ("embedding", 1000, 768, 257),
                     ("embedding", 700, 100, 40), ("tiny", 300, 37, 20), ("deep", 3000, 96, 1000)]


@pytest.mark.parametrize("gen,n,d,k", CASES_BF16_SEARCH)
def test_assign_bf16_search(mm, gen, n, d, k):
    """fp32 rows searched in bf16: the oracle's assignment of the bf16-rounded
    rows against the bf16-rounded centroids."""
    import torch
    X = datagen.make(gen, n, d, seed=17)
    C = _centroids(X, k, 8)
    lab, dist = mm.assign(to_device(X), torch.from_numpy(C).cuda(), bf16_search=True)
    lab, dist = lab.cpu().numpy(), dist.cpu().numpy()
    Xs = oracle.Converter("bf16").rows(X)
    Cs = oracle.bf16_round(C)
    olab, d1, d2 = oracle.assign(Xs, Cs)
    check_labels(Xs, Cs, None, lab, olab, d1, d2, what=f"bf16-search {gen} {n}x{d} k={k}")
    check_dists(Xs, Cs, None, lab, dist, what=f"bf16-search {gen} {n}x{d} k={k}")


CASES_SPHERICAL = [("embedding", 1500, 768, 300, False), ("deep", 3000, 96, 1000, False),
                   ("tiny", 700, 16, 40, False), ("large", 2000, 128, 300, True),
                   ("large", 900, 64, 129, True), ("large", 600, 256, 70, True),
                   ("large", 1100, 768, 65, True)]


def _unit_rows(A):
    A = A.astype(np.float64)
    return (A / np.maximum(np.linalg.norm(A, axis=1, keepdims=True), 1e-30)).astype(np.float32)


@pytest.mark.parametrize("gen,n,d,k,bf16", CASES_SPHERICAL)
def test_assign_spherical(mm, gen, n, d, k, bf16):
    """README "Spherical e-means": the centroid of largest dot product and
    that similarity (a zero centroid included, which scores 0)."""
    import torch
    X = datagen.make(gen, n, d, seed=19)
    if not bf16:
        X = _unit_rows(X)
    C = _unit_rows(_centroids(X, k, 9))
    C[k // 2] = 0.0
    lab, sim = mm.assign(to_device(X), torch.from_numpy(C).cuda(), spherical=True)
    lab, sim = lab.cpu().numpy(), sim.cpu().numpy()
    Cs = oracle.bf16_round(C) if bf16 else C
    olab, s1, s2 = oracle.assign_ip(X, Cs)
    gd = -2.0 * oracle.dot_to(X, Cs, lab)
    check_labels(X, Cs, None, lab, olab, -2.0 * s1, -2.0 * s2, given_dist=gd,
                 what=f"spherical {gen} {n}x{d} k={k}")
    ref = oracle.dot_to(X, Cs, lab)
    Xf = oracle.to_f32(X).astype(np.float64)
    scale = np.einsum("ij,ij->i", Xf, Xf) + np.sum(Cs[lab].astype(np.float64) ** 2, axis=1)
    assert np.all(np.abs(sim - ref) <= 1e-5 * scale)


CASES_I8 = [(2000, 768, 300), (1000, 64, 129), (777, 48, 50), (500, 37, 20), (300, 256, 1),
            (900, 520, 300), (600, 1040, 257), (3000, 128, 1000),
            # d = 32..256 in steps of 32 take the register-resident kernel:
            # every k-step count, several workgroups with a ragged last one,
            # k past one 256-centroid panel and not a multiple of 32
            (1500, 32, 513), (2049, 96, 300), (2500, 160, 700), (1100, 192, 33),
            (2100, 224, 290), (1700, 256, 600),
            # d = 512 and 768 take the wide resident kernel (64 points per
            # wave, 64-centroid panels): one panel, a ragged panel and point
            # tile, k = 1, several workgroups with a ragged last one
            (256, 512, 64), (777, 512, 65), (4097, 768, 1025), (300, 768, 1),
            (1300, 768, 129)]


def _int8_centroids(X, k, seed):
    """Code-space centroids near data rows, a few coordinates outside the code
    range (clamped to +-127) and at exact half-integers (ties to even)."""
    C = _centroids(X, k, seed)
    d = C.shape[1]
    C[0, : min(d, 4)] = np.array([200.0, -300.0, 126.5, -0.5], np.float32)[: min(d, 4)]
    if k > 1:
        C[1, : min(d, 2)] = np.array([2.5, -127.5], np.float32)[: min(d, 2)]
    return C


@pytest.mark.parametrize("n,d,k", CASES_I8)
def test_assign_int8(mm, n, d, k):
    """int8 codes: the search is exact in integers, so labels (lowest index on
    ties) and distances equal the oracle's exactly."""
    X = datagen.codes_i8(n, d, m=64, seed=23)
    C = _int8_centroids(X, k, 10)
    lab, dist = _run(mm, X, C)
    Cs = oracle.int8_round(C)
    olab, d1, _ = oracle.assign(X, Cs)
    assert np.array_equal(lab, olab), f"{int(np.sum(lab != olab))} labels differ"
    assert np.array_equal(dist, d1.astype(np.float32))


def test_assign_int8_misaligned(mm):
    """Rows that do not start on a 16-byte boundary take the register-staged
    kernel; the result is the same exact assignment."""
    import torch
    n, d, k = 700, 64, 90
    X = datagen.codes_i8(n, d, m=32, seed=29)
    C = _int8_centroids(X, k, 12)
    buf = torch.empty(n * d + 1, dtype=torch.int8, device="cuda")
    Xd = buf[1:].view(n, d)
    Xd.copy_(torch.from_numpy(X).cuda())
    lab, dist = mm.assign(Xd, torch.from_numpy(C).cuda())
    olab, d1, _ = oracle.assign(X, oracle.int8_round(C))
    assert np.array_equal(lab.cpu().numpy(), olab)
    assert np.array_equal(dist.cpu().numpy(), d1.astype(np.float32))


def test_assign_int8_rules(mm):
    import torch
    X = torch.zeros((10, 43920), dtype=torch.int8, device="cuda")
    C = torch.zeros((2, 43920), dtype=torch.float32, device="cuda")
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        mm.assign(X, C)
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        mm.assign(X[:, :16].contiguous(), C[:, :16].contiguous(), spherical=True)


CASES_U8 = [(2000, 768, 300), (1000, 64, 129), (777, 48, 50), (500, 37, 20), (300, 256, 1),
            (600, 1040, 257), (3000, 128, 1000),
            (1500, 32, 513), (2049, 96, 300), (2500, 160, 700), (1100, 192, 33),
            (2100, 224, 290), (1700, 256, 600),
            (777, 512, 65), (4097, 768, 1025), (300, 768, 1)]


def _u8_centroids(X, k, seed):
    """Centroids near data rows, a few coordinates outside [0, 255] (clamped)
    and at exact half-integers (ties to even)."""
    C = _centroids(X, k, seed)
    d = C.shape[1]
    C[0, : min(d, 4)] = np.array([300.0, -20.0, 254.5, 0.5], np.float32)[: min(d, 4)]
    if k > 1:
        C[1, : min(d, 2)] = np.array([2.5, 255.5], np.float32)[: min(d, 2)]
    return C


@pytest.mark.parametrize("n,d,k", CASES_U8)
def test_assign_uint8(mm, n, d, k):
    """uint8 data: the search is exact in integers, so labels (lowest index on
    ties) and distances equal the oracle's exactly."""
    X = datagen.codes_u8(n, d, m=64, seed=37).view(oracle.U8)
    C = _u8_centroids(X, k, 15)
    lab, dist = _run(mm, X, C)
    olab, d1, _ = oracle.assign(X, oracle.u8_round(C))
    assert np.array_equal(lab, olab), f"{int(np.sum(lab != olab))} labels differ"
    assert np.array_equal(dist, d1.astype(np.float32))


@pytest.mark.parametrize("d", [43919, 43904])
def test_assign_uint8_extremes_at_the_dimension_limit(mm, d):
    """Rows of 0s, 255s and 128s against centroids of 0s and 255s at the
    largest d: the losing score of a 255-row against the 0-centroid is
    -48896 d, one step from the int32 limit; labels and distances stay exact
    (d = 43904: whole 16-byte rows; 43919: the unaligned tail)."""
    raw = np.zeros((3, d), np.uint8)
    raw[1] = 255
    raw[2] = 128
    C = np.zeros((2, d), np.float32)
    C[1] = 255.0
    X = raw.view(oracle.U8)
    lab, dist = _run(mm, X, C)
    olab, d1, _ = oracle.assign(X, oracle.u8_round(C))
    assert lab.tolist() == [0, 1, 1] and np.array_equal(lab, olab)   # 128 is nearer 255
    assert np.array_equal(dist, d1.astype(np.float32))


def test_assign_uint8_misaligned_and_rules(mm):
    import torch
    n, d, k = 700, 64, 90
    X = datagen.codes_u8(n, d, m=32, seed=39).view(oracle.U8)
    C = _u8_centroids(X, k, 16)
    buf = torch.empty(n * d + 1, dtype=torch.uint8, device="cuda")
    Xd = buf[1:].view(n, d)
    Xd.copy_(torch.from_numpy(X.view(np.uint8)).cuda())
    lab, dist = mm.assign(Xd, torch.from_numpy(C).cuda())
    olab, d1, _ = oracle.assign(X, oracle.u8_round(C))
    assert np.array_equal(lab.cpu().numpy(), olab)
    assert np.array_equal(dist.cpu().numpy(), d1.astype(np.float32))
    Z = torch.zeros((10, 43920), dtype=torch.uint8, device="cuda")
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        mm.assign(Z, torch.zeros((2, 43920), device="cuda"))
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        mm.assign(Xd, torch.from_numpy(C).cuda(), spherical=True)


CASES_F8 = [(2000, 768, 300), (1000, 64, 129), (777, 48, 50), (500, 37, 20), (300, 256, 1),
            (600, 1040, 257), (3000, 128, 1000),
            # the register-resident kernel of d = 512 and 768: ragged point
            # tiles (256 per workgroup) and ragged 64-row centroid panels
            (4097, 512, 1025), (300, 512, 1), (1300, 768, 129), (257, 768, 64)]


@pytest.mark.parametrize("n,d,k", CASES_F8)
def test_assign_fp8(mm, n, d, k):
    """FP8 E4M3 codes: the search uses the centroids rounded to E4M3 (ties to
    even, saturating; a few coordinates set past the range and on ties)."""
    X = datagen.codes_e4m3(n, d, m=64, seed=25)
    C = _centroids(X, k, 11)
    C[0, : min(d, 4)] = np.array([500.0, -1e4, 1.0625, -1.1875], np.float32)[: min(d, 4)]
    lab, dist = _run(mm, X, C)
    Cs = oracle.e4m3_round(C)
    olab, d1, d2 = oracle.assign(X, Cs)
    check_labels(X, Cs, None, lab, olab, d1, d2, what=f"fp8 {n}x{d} k={k}")
    check_dists(X, Cs, None, lab, dist, what=f"fp8 {n}x{d} k={k}")


def test_assign_fp8_misaligned_and_rules(mm):
    import torch
    n, d, k = 700, 64, 90
    X = datagen.codes_e4m3(n, d, m=32, seed=29)
    C = _centroids(X, k, 12)
    buf = torch.empty(n * d + 1, dtype=torch.uint8, device="cuda")
    Xd = buf[1:].view(n, d)
    Xd.copy_(torch.from_numpy(X).cuda())
    lab, dist = mm.assign(Xd.view(torch.float8_e4m3fn), torch.from_numpy(C).cuda())
    Cs = oracle.e4m3_round(C)
    olab, d1, d2 = oracle.assign(X, Cs)
    check_labels(X, Cs, None, lab.cpu().numpy(), olab, d1, d2, what="fp8 misaligned")
    with pytest.raises(mm.EmeansError, match="EINVAL"):
        mm.assign(to_device(X), torch.from_numpy(C).cuda(), spherical=True)


@pytest.mark.parametrize("n,d,k", CASES_BF16)
def test_assign_bf16(mm, n, d, k):
    X = datagen.large_host(n, d=d, m=64, seed=13)
    C = _centroids(X, k, 6)
    lab, dist = _run(mm, X, C)
    Cs = oracle.bf16_round(C)                # bf16 data is searched with bf16 centroids
    olab, d1, d2 = oracle.assign(X, Cs)
    check_labels(X, Cs, None, lab, olab, d1, d2, what=f"bf16 {n}x{d} k={k}")
    check_dists(X, Cs, None, lab, dist, what=f"bf16 {n}x{d} k={k}")


@pytest.mark.parametrize("n,k,sph", [((1 << 20) + 77, 1000, False), (1 << 20, 129, True)])
def test_assign_bf16_large_batch(mm, n, k, sph):
    """A batch of more than 2^20 bf16 rows of d = 128 (the 100M-row set's
    batch scale) in the register-resident kernel: a ragged last point tile
    and a ragged last centroid panel, checked on a sample of rows and on the
    last rows of the batch (and in spherical mode, the similarity)."""
    import torch
    X = datagen.large_host(n, d=128, m=64, seed=17)
    C = _centroids(X[:65536], k, 8)
    if sph:
        C = (C / np.linalg.norm(C.astype(np.float64), axis=1, keepdims=True)).astype(np.float32)
    lab, dist = mm.assign(to_device(X), torch.from_numpy(C).cuda(), spherical=sph)
    lab, dist = lab.cpu().numpy(), dist.cpu().numpy()
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(n, 3000, replace=False),
                                     np.arange(n - 300, n)]))
    Cs = oracle.bf16_round(C)
    what = f"bf16 large batch {n}x128 k={k}{' spherical' if sph else ''}"
    if sph:
        olab, s1, s2 = oracle.assign_ip(X, Cs, rows)
        ref = oracle.dot_to(X, Cs, lab[rows], rows)
        check_labels(X, Cs, rows, lab[rows], olab, -2.0 * s1, -2.0 * s2, given_dist=-2.0 * ref,
                     what=what)
        Xf = oracle.to_f32(X[rows]).astype(np.float64)
        scale = np.einsum("ij,ij->i", Xf, Xf) + np.sum(Cs[lab[rows]].astype(np.float64) ** 2, axis=1)
        assert np.all(np.abs(dist[rows] - ref) <= 1e-5 * scale)
    else:
        olab, d1, d2 = oracle.assign(X, Cs, rows)
        check_labels(X, Cs, rows, lab[rows], olab, d1, d2, what=what)
        check_dists(X, Cs, rows, lab[rows], dist[rows], what=what)
    assert lab.min() >= 0 and lab.max() < k


CASES_F16 = [("embedding", 2000, 768, 300), ("deep", 1000, 96, 129), ("sift", 1500, 128, 257),
             ("tiny", 777, 40, 50), ("tiny", 500, 37, 20), ("embedding", 300, 256, 1),
             ("deep", 600, 32, 70), ("sift", 900, 64, 1000), ("embedding", 513, 1040, 257),
             ("embedding", 4097, 768, 1025)]


@pytest.mark.parametrize("gen,n,d,k", CASES_F16)
def test_assign_fp16(mm, gen, n, d, k):
    """fp16 data (README "Data precision", FP16) is searched with the
    centroids rounded to fp16; d = 32, 64, 96 and 128 take the kernel that
    keeps the points in registers, d = 37 the unaligned path."""
    X = datagen.make(gen + "-f16", n, d, seed=27)
    C = _centroids(X, k, 13)
    lab, dist = _run(mm, X, C)
    Cs = oracle.f16_round(C)
    olab, d1, d2 = oracle.assign(X, Cs)
    check_labels(X, Cs, None, lab, olab, d1, d2, what=f"fp16 {gen} {n}x{d} k={k}")
    check_dists(X, Cs, None, lab, dist, what=f"fp16 {gen} {n}x{d} k={k}")


def test_assign_fp16_rounding_and_misaligned(mm):
    """The search centroid is the nearest fp16 value (ties to even, subnormals
    kept, 65519 down to 65504): from a zero row the distance is exactly the
    square of the rounded coordinate. Then a view at an odd element offset."""
    import torch
    vals = [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -(1 + 2.0 ** -11), 65519.0, 1.5 * 2.0 ** -24,
            3 * 2.0 ** -20, 0.1, -2049.0, 2051.0]
    for d in (1, 8):
        for v in vals:
            C = np.zeros((1, d), np.float32)
            C[0, 0] = v
            lab, dist = _run(mm, np.zeros((3, d), np.float16), C)
            want = np.float32(oracle.f16_round(np.float32(v))) ** 2
            assert lab.tolist() == [0, 0, 0] and np.all(dist == want), (d, v, dist, want)
    n, d, k = 700, 64, 90
    X = datagen.make("embedding-f16", n, d, seed=29)
    C = _centroids(X, k, 12)
    buf = torch.empty(n * d + 1, dtype=torch.float16, device="cuda")
    Xd = buf[1:].view(n, d)
    Xd.copy_(torch.from_numpy(X).cuda())
    lab, dist = mm.assign(Xd, torch.from_numpy(C).cuda())
    Cs = oracle.f16_round(C)
    olab, d1, d2 = oracle.assign(X, Cs)
    check_labels(X, Cs, None, lab.cpu().numpy(), olab, d1, d2, what="fp16 misaligned")
    check_dists(X, Cs, None, lab.cpu().numpy(), dist.cpu().numpy(), what="fp16 misaligned")


@pytest.mark.parametrize("n,d,k", [(1500, 768, 300), (3000, 96, 1000), (900, 128, 257)])
def test_assign_fp16_spherical(mm, n, d, k):
    """Spherical e-means on fp16 data: highest dot product with the unit
    centroids rounded to fp16, and that similarity."""
    import torch
    X = _unit_rows(datagen.make("embedding", n, d, seed=31)).astype(np.float16)
    C = _unit_rows(_centroids(X, k, 14))
    lab, sim = mm.assign(to_device(X), torch.from_numpy(C).cuda(), spherical=True)
    lab, sim = lab.cpu().numpy(), sim.cpu().numpy()
    Cs = oracle.f16_round(C)
    olab, s1, s2 = oracle.assign_ip(X, Cs)
    gd = -2.0 * oracle.dot_to(X, Cs, lab)
    check_labels(X, Cs, None, lab, olab, -2.0 * s1, -2.0 * s2, given_dist=gd,
                 what=f"spherical fp16 {n}x{d} k={k}")
    Xf = oracle.to_f32(X).astype(np.float64)
    scale = np.einsum("ij,ij->i", Xf, Xf) + np.sum(Cs[lab].astype(np.float64) ** 2, axis=1)
    assert np.all(np.abs(sim - oracle.dot_to(X, Cs, lab)) <= 1e-5 * scale)


def test_assign_ties_lowest_index(mm):
    rng = np.random.default_rng(3)
    X = rng.standard_normal((500, 24)).astype(np.float32)
    base = rng.standard_normal((40, 24)).astype(np.float32)
    C = np.concatenate([base, base, base[:7]])  # exact duplicates: the first copy must win
    lab, _ = _run(mm, X, C)
    olab, _, _ = oracle.assign(X, C)
    assert np.array_equal(lab, olab)
    assert lab.max() < 40


def test_assign_exact_hits(mm):
    """Rows equal to a centroid get that centroid and distance ~0."""
    X = datagen.sift(n=600, d=128, seed=2)
    C = np.ascontiguousarray(X[::7][:80])
    lab, dist = _run(mm, X, C)
    hit = np.arange(0, 600, 7)[:80]
    assert np.array_equal(lab[hit], oracle.assign(X[hit], C)[0])
    assert np.all(dist[hit] <= 1e-5 * 2 * np.einsum("ij,ij->i", X[hit], X[hit]))


def test_assign_empty_and_single(mm):
    import torch
    X = torch.zeros((0, 8), device="cuda")
    lab, dist = mm.assign(X, torch.zeros((3, 8), device="cuda"))
    assert lab.numel() == 0
    Xs = datagen.tiny(n=1, d=8)
    C = _centroids(datagen.tiny(n=50, d=8), 5, 1)
    lab, _ = _run(mm, Xs, C)
    assert lab[0] == oracle.assign(Xs, C)[0][0]


def test_assign_rejects_bad_args(mm):
    import torch
    with pytest.raises(mm.EmeansError):
        mm.assign(torch.zeros((10, 4), device="cuda", dtype=torch.float64),
                  torch.zeros((3, 4), device="cuda"))
    with pytest.raises(mm.EmeansError):
        mm.assign(torch.zeros((10, 4), device="cuda"), torch.zeros((3, 5), device="cuda"))


@pytest.mark.parametrize("n", [1, 2, 10, 1000, 10007, 65536, 1_000_000])
def test_batch_rows_bit_exact(mm, n):
    seed = 1234
    for pass_ in (0, 3):
        count = min(n, 50_000)
        start = (n - count) // 2
        got = mm.batch_rows(n, seed, pass_, start, count).cpu().numpy()
        want = oracle.perm_range(n, seed, oracle.STREAM_PERM, pass_, start, count)
        assert np.array_equal(got, want)
    if n <= 65536:
        full = mm.batch_rows(n, seed, 1, 0, n).cpu().numpy()
        assert np.array_equal(np.sort(full), np.arange(n))


@pytest.mark.parametrize("u8", [False, True])
@pytest.mark.parametrize("d", [64, 160])
def test_assign_integer_ties_take_the_lowest_index(mm, u8, d):
    """Copies of one centroid at indices that fall in the two lane halves of a
    32-centroid block, in different blocks and in different 256-centroid
    panels: every point nearest to that centroid takes its lowest index."""
    n, k = 1200, 700
    if u8:
        X = datagen.codes_u8(n, d, m=16, seed=41).view(oracle.U8)
        C = _u8_centroids(X, k, 16)
    else:
        X = datagen.codes_i8(n, d, m=16, seed=41)
        C = _int8_centroids(X, k, 16)
    Xf = oracle.to_f32(X)
    for src, dups in ((3, (7, 12, 40, 300, 699)), (5, (4,)), (600, (601, 33))):
        C[list(dups)] = C[src]
    for j, row in ((20, 0), (21, 1), (290, 2)):  # centroids on data rows: exact hits
        C[j] = Xf[row]
    C[[520, 260, 9]] = Xf[0]
    lab, dist = _run(mm, X, C)
    Cs = oracle.u8_round(C) if u8 else oracle.int8_round(C)
    olab, d1, _ = oracle.assign(X, Cs)
    assert np.array_equal(lab, olab), f"{int(np.sum(lab != olab))} labels differ"
    assert np.array_equal(dist, d1.astype(np.float32))


@pytest.mark.parametrize("u8", [False, True])
@pytest.mark.parametrize("n", [70_000, 140_000, 270_000])
def test_assign_integer_batch_sizes(mm, u8, n):
    """The register-resident integer kernel splits the 32-centroid blocks of
    a panel among 8 waves for small batches (the cases above), among 4 and 2
    waves at 70000 and 140000 rows of d = 64, and not at all at 270000 rows:
    every split gives the same exact result."""
    d, k = 64, 333
    if u8:
        X = datagen.codes_u8(n, d, m=64, seed=43).view(oracle.U8)
        C = _u8_centroids(X, k, 17)
        Cs = oracle.u8_round(C)
    else:
        X = datagen.codes_i8(n, d, m=64, seed=43)
        C = _int8_centroids(X, k, 17)
        Cs = oracle.int8_round(C)
    lab, dist = _run(mm, X, C)
    olab, d1, _ = oracle.assign(X, Cs)
    assert np.array_equal(lab, olab), f"{int(np.sum(lab != olab))} labels differ"
    assert np.array_equal(dist, d1.astype(np.float32))
