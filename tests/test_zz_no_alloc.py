"""emeans_assign_static: the nearest-centroid search with no memory
allocation (its working memory is one fixed device array per GPU), for
callers that cannot allocate. Its results must equal emeans_assign's, which
runs the same kernels on allocated memory: labels and distances bit for bit,
on two calls in a row (the second smaller, so stale contents of the shared
array from the first call would show), for each search format that uses the
array differently."""
import re

import pytest

from mini_means_amd import datagen

from parity import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mm():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mini_means_amd
    mini_means_amd.lib()
    return mini_means_amd


def scratch_bytes(mm):
    with open(mm.HEADER) as f:
        return int(eval(re.search(r"#define EMEANS_STATIC_SCRATCH_BYTES \((.*)\)", f.read())
                        .group(1).replace("u", "")))


# (name, generator, [(n, d, k), (smaller n, d, k)], options)
CASES = [
    ("f32-768", "embedding", [(20_000, 768, 4096), (5_000, 768, 1000)], {}),
    ("bf16-large-k", "large", [(30_000, 128, 65536), (4_000, 128, 5000)], {}),
    ("f16-search", "deep", [(20_000, 96, 512), (3_001, 96, 77)], dict(search="f16")),
    ("bf16-search-sph", "embedding", [(8_000, 768, 1024), (999, 768, 300)],
     dict(bf16_search=True, spherical=True)),
    ("int8", "codes", [(10_000, 64, 256), (1_234, 64, 50)], {}),
    ("u8", "codes-u8", [(10_000, 128, 512), (2_000, 128, 64)], {}),
]


@pytest.mark.parametrize("name,gen,shapes,o", CASES, ids=[c[0] for c in CASES])
def test_static_assign_equals_assign(mm, name, gen, shapes, o):
    import torch
    for call, (n, d, k) in enumerate(shapes):
        print(f"[no-alloc] {name} call {call}: n={n} d={d} k={k}", flush=True)
        X = datagen.make(gen, n, d, seed=31 + call)
        Xd = to_device(X)
        # centroids: other rows of the same generator, as fp32 values
        Cd = to_device(datagen.make(gen, k, d, seed=41 + call)).float().contiguous()
        if o.get("spherical"):
            Cd = torch.nn.functional.normalize(Cd, dim=1).contiguous()
        ref_l, ref_d = mm.assign(Xd, Cd, **o)
        lab = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        dst = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        got_l, got_d = mm.assign(Xd, Cd, no_alloc=True, out=(lab, dst), **o)
        torch.cuda.synchronize()
        assert torch.equal(got_l, ref_l), f"{name}: labels differ on call {call}"
        assert torch.equal(got_d, ref_d), f"{name}: distances differ on call {call}"


def test_static_assign_rejects_beyond_its_array(mm):
    """A bf16 search copy of k x d larger than the array fails with EINVAL
    before any work; a size that fits still runs."""
    import torch
    cap = scratch_bytes(mm)
    d = 128
    k = cap // (2 * d) + 1                  # the k x d bf16 copy alone exceeds it
    X = torch.zeros((16, d), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((k, d), dtype=torch.float32, device="cuda")
    with pytest.raises(mm.EmeansError, match="EINVAL.*scratch"):
        mm.assign(X, C, no_alloc=True)
    lab, dist = mm.assign(X, C[:1000].contiguous(), no_alloc=True)
    assert torch.all(lab == 0) and torch.all(dist == 0)
