"""Seeded synthetic inputs for the e-means workloads.

This module only draws data. It contains none of the clustering arithmetic and
is shared by the tests, the benchmark and the CPU checker so that every side
reads the same bytes. Each generator is deterministic in (seed, split) and in
the row count, independent of how many threads generate it: rows are produced
in fixed chunks, each chunk with its own PCG64 stream keyed by
(seed, stream, chunk index).

The workloads stand in for the datasets the e-means pages measure on (several
embedding sets, DEEP1M, SIFT, 100M-scale runs), none of which is available
here:

* ``tiny``       n=10,000, d=16, mixture of 64 isotropic Gaussians, centres
                 N(0, I), sigma 0.3, equal weights.
* ``embedding``  d=768, 4,096-component mixture, Zipf(1.1) weights, centres
                 N(0, I), per-coordinate noise 0.5, then unit-normalised.
* ``deep``       d=96, rank-32 Gaussian W z (W entries N(0, 1/32)) plus
                 isotropic noise 0.1, then unit-normalised.
* ``sift``       d=128, each coordinate 0 with probability 0.3, else
                 clip(round(|N(0, 40^2)|), 0, 255); stored as fp32 integers.
* ``large``      d=128, 65,536 equal-weight components, centres N(0, I),
                 noise 0.4, unit-normalised, rounded to bf16. Generated on the
                 GPU with torch's seeded generator (25.6 GB at n=1e8).

``split=0`` is the training set, ``split=1`` the held-out set drawn from the
same mixture (same centres, different sample stream).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 15  # rows per independently seeded chunk


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(v) for v in key]))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(n: int, d: int, dtype, fill) -> np.ndarray:
    """Allocate n x d and fill it chunk by chunk; fill(c, lo, hi, out_view)."""
    out = np.empty((n, d), dtype=dtype)
    spans = [(c, lo, min(n, lo + CHUNK)) for c, lo in enumerate(range(0, n, CHUNK))]
    if len(spans) <= 1:
        for c, lo, hi in spans:
            fill(c, lo, hi, out[lo:hi])
        return out
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda s: fill(s[0], s[1], s[2], out[s[1]:s[2]]), spans))
    return out


def _normalize_rows(x: np.ndarray) -> np.ndarray:
    nrm = np.sqrt(np.einsum("ij,ij->i", x.astype(np.float64), x.astype(np.float64)))
    nrm[nrm == 0] = 1.0
    return (x / nrm[:, None].astype(np.float32)).astype(np.float32)


# ----------------------------------------------------------------------------
# generators (host)
# ----------------------------------------------------------------------------

def tiny(n: int = 10_000, d: int = 16, m: int = 64, sigma: float = 0.3,
         seed: int = 101, split: int = 0) -> np.ndarray:
    means = _rng(seed, 0).standard_normal((m, d)).astype(np.float32)

    def fill(c, lo, hi, out):
        r = _rng(seed, 1 + split, c)
        comp = r.integers(0, m, size=hi - lo)
        g = r.standard_normal((hi - lo, d), dtype=np.float32)
        out[:] = means[comp] + np.float32(sigma) * g

    return _chunked(n, d, np.float32, fill)


def zipf_weights(m: int, s: float) -> np.ndarray:
    w = np.arange(1, m + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def embedding(n: int = 1_000_000, d: int = 768, m: int = 4096, zipf: float = 1.1,
              sigma: float = 0.5, seed: int = 102, split: int = 0) -> np.ndarray:
    means = _rng(seed, 0).standard_normal((m, d)).astype(np.float32)
    cdf = np.cumsum(zipf_weights(m, zipf))
    cdf[-1] = 1.0

    def fill(c, lo, hi, out):
        r = _rng(seed, 1 + split, c)
        comp = np.searchsorted(cdf, r.random(hi - lo), side="right")
        comp = np.minimum(comp, m - 1)
        g = r.standard_normal((hi - lo, d), dtype=np.float32)
        out[:] = _normalize_rows(means[comp] + np.float32(sigma) * g)

    return _chunked(n, d, np.float32, fill)


def deep(n: int = 1_000_000, d: int = 96, rank: int = 32, sigma: float = 0.1,
         seed: int = 103, split: int = 0) -> np.ndarray:
    W = (_rng(seed, 0).standard_normal((d, rank)) / np.sqrt(rank)).astype(np.float32)

    def fill(c, lo, hi, out):
        r = _rng(seed, 1 + split, c)
        z = r.standard_normal((hi - lo, rank), dtype=np.float32)
        g = r.standard_normal((hi - lo, d), dtype=np.float32)
        out[:] = _normalize_rows(z @ W.T + np.float32(sigma) * g)

    return _chunked(n, d, np.float32, fill)


def sift(n: int = 1_000_000, d: int = 128, scale: float = 40.0, p_zero: float = 0.3,
         seed: int = 104, split: int = 0) -> np.ndarray:
    def fill(c, lo, hi, out):
        r = _rng(seed, 1 + split, c)
        v = np.clip(np.rint(np.abs(r.standard_normal((hi - lo, d)) * scale)), 0, 255)
        v[r.random((hi - lo, d)) < p_zero] = 0.0
        out[:] = v.astype(np.float32)

    return _chunked(n, d, np.float32, fill)


def large_means(m: int = 65536, d: int = 128, seed: int = 105) -> np.ndarray:
    return _rng(seed, 0).standard_normal((m, d)).astype(np.float32)


def large_host(n: int, d: int = 128, m: int = 65536, sigma: float = 0.4,
               seed: int = 105, split: int = 0) -> np.ndarray:
    """Host version of the Large generator for small n; returns bf16 bits (uint16).

    Same mixture as ``large_device`` but a different sample stream: used for
    small-n tests that do not need a GPU to create data.
    """
    means = large_means(m, d, seed)

    def fill(c, lo, hi, out):
        r = _rng(seed, 1 + split, c)
        comp = r.integers(0, m, size=hi - lo)
        g = r.standard_normal((hi - lo, d), dtype=np.float32)
        out[:] = f32_to_bf16_bits(_normalize_rows(means[comp] + np.float32(sigma) * g))

    return _chunked(n, d, np.uint16, fill)


def large_device(n: int = 100_000_000, d: int = 128, m: int = 65536, sigma: float = 0.4,
                 seed: int = 105, split: int = 0, device: str = "cuda:0"):
    """The Large workload generated on the GPU (torch.bfloat16 tensor, n x d).

    Centres come from the host PCG64 stream; component ids and noise from
    torch's seeded device generator, in fixed chunks of 2^20 rows.
    """
    import torch

    means = torch.from_numpy(large_means(m, d, seed)).to(device)
    out = torch.empty((n, d), dtype=torch.bfloat16, device=device)
    gen = torch.Generator(device=device)
    step = 1 << 20
    for c, lo in enumerate(range(0, n, step)):
        hi = min(n, lo + step)
        gen.manual_seed(int(seed) * 1_000_003 + 7919 * (1 + split) + c)
        comp = torch.randint(0, m, (hi - lo,), generator=gen, device=device)
        g = torch.randn((hi - lo, d), generator=gen, device=device, dtype=torch.float32)
        x = means[comp] + sigma * g
        x = x / x.norm(dim=1, keepdim=True).clamp_min(1e-30)
        out[lo:hi] = x.to(torch.bfloat16)
    return out


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# named workloads
# ----------------------------------------------------------------------------

WORKLOADS = {
    # name: (generator, kwargs, k, T, dtype, held-out rows)
    "tiny": dict(gen="tiny", n=10_000, d=16, k=64, T=5.0, dtype="f32", heldout=10_000),
    "embedding": dict(gen="embedding", n=1_000_000, d=768, k=4096, T=5.0, dtype="f32",
                      heldout=100_000),
    "deep": dict(gen="deep", n=1_000_000, d=96, k=16384, T=5.0, dtype="f32", heldout=100_000),
    "sift": dict(gen="sift", n=1_000_000, d=128, k=16384, T=5.0, dtype="f32", heldout=100_000),
    "large": dict(gen="large", n=100_000_000, d=128, k=65536, T=3.0, dtype="bf16",
                  heldout=1_000_000),
}


def codes_i8(n: int = 1_000_000, d: int = 768, m: int = 4096, spread: float = 80.0,
             sigma: float = 12.0, seed: int = 107, split: int = 0) -> np.ndarray:
    """int8 codes of clustered data (README "Data precision", INT8 input):
    m centres uniform in [-spread, spread]^d, Zipf(1.1) weights, Gaussian
    noise of s.d. sigma, rounded to the nearest integer and clamped to
    [-127, 127] (a few values saturate, as real calibrated codes do)."""
    r0 = _rng(seed, 0)
    means = r0.uniform(-spread, spread, size=(m, d)).astype(np.float32)
    w = zipf_weights(m, 1.1)

    def fill(c, lo, hi, out):
        r = _rng(seed, 1 + split, c)
        comp = r.choice(m, size=hi - lo, p=w)
        g = r.standard_normal((hi - lo, d), dtype=np.float32)
        out[:] = np.clip(np.rint(means[comp] + np.float32(sigma) * g), -127, 127).astype(np.int8)

    return _chunked(n, d, np.int8, fill)


# uint8 data is handed to the oracle as `raw.view(U8)`: a one-field structured
# dtype over the same bytes (plain numpy uint8 stands for E4M3 bit patterns).
U8 = np.dtype([("u8", np.uint8)])


def codes_u8(n: int = 1_000_000, d: int = 128, m: int = 4096, lo: float = 40.0,
             hi: float = 215.0, sigma: float = 12.0, seed: int = 111,
             split: int = 0) -> np.ndarray:
    """uint8 data with clusters (README "Data precision", UINT8 input, e.g.
    raw descriptor bytes): m centres uniform in [lo, hi]^d, Zipf(1.1) weights,
    Gaussian noise of s.d. sigma, rounded and clamped to [0, 255]. Returns
    the raw bytes (numpy uint8); `make` marks them with U8."""
    r0 = _rng(seed, 0)
    means = r0.uniform(lo, hi, size=(m, d)).astype(np.float32)
    w = zipf_weights(m, 1.1)

    def fill(c, lo_, hi_, out):
        r = _rng(seed, 1 + split, c)
        comp = r.choice(m, size=hi_ - lo_, p=w)
        g = r.standard_normal((hi_ - lo_, d), dtype=np.float32)
        out[:] = np.clip(np.rint(means[comp] + np.float32(sigma) * g), 0, 255).astype(np.uint8)

    return _chunked(n, d, np.uint8, fill)


def codes_e4m3(n: int = 1_000_000, d: int = 768, m: int = 1024, sigma: float = 2.0,
               seed: int = 109, split: int = 0) -> np.ndarray:
    """FP8 E4M3 codes of clustered data (README "Data precision", FP8 input),
    drawn directly as bit patterns: each of m centres has, per dimension, a
    sign bit and a magnitude code in [24, 112] (E4M3 codes grow with the
    value, so nearby codes are nearby values); a row of a centre keeps its
    signs and moves each magnitude code by a rounded Gaussian of s.d. sigma,
    clamped to [0, 126] (126 = 0x7E, the largest finite code). Zipf(1.1)
    weights."""
    r0 = _rng(seed, 0)
    mag = r0.integers(24, 113, size=(m, d))
    sgn = r0.integers(0, 2, size=(m, d)) * 0x80
    w = zipf_weights(m, 1.1)

    def fill(c, lo, hi, out):
        r = _rng(seed, 1 + split, c)
        comp = r.choice(m, size=hi - lo, p=w)
        noise = np.rint(r.standard_normal((hi - lo, d)) * sigma).astype(np.int64)
        out[:] = (sgn[comp] | np.clip(mag[comp] + noise, 0, 126)).astype(np.uint8)

    return _chunked(n, d, np.uint8, fill)


def make(gen: str, n: int, d: int, split: int = 0, **kw) -> np.ndarray:
    """Host data for a generator name at any (n, d) (fp32, bf16 bits for
    'large', int8 for 'codes', E4M3 bits for 'codes8', U8-marked bytes for
    'codes-u8' and 'sift-u8'). A name ending in '-f16' stores that generator's
    rows as IEEE fp16 (numpy float16: nearest, ties to even), the one-off
    conversion a caller makes for FP16 data."""
    if gen == "codes-u8":
        return codes_u8(n=n, d=d, split=split, **kw).view(U8)
    if gen == "sift-u8":   # the SIFT-like values are integers in [0, 255]
        return sift(n=n, d=d, split=split, **kw).astype(np.uint8).view(U8)
    if gen.endswith("-f16"):
        X = make(gen[:-4], n, d, split=split, **kw)
        if X.dtype == np.uint16:
            X = bf16_bits_to_f32(X)
        return X.astype(np.float16)
    if gen == "codes":
        return codes_i8(n=n, d=d, split=split, **kw)
    if gen == "codes8":
        return codes_e4m3(n=n, d=d, split=split, **kw)
    if gen == "tiny":
        return tiny(n=n, d=d, split=split, **kw)
    if gen == "embedding":
        return embedding(n=n, d=d, split=split, **kw)
    if gen == "deep":
        return deep(n=n, d=d, split=split, **kw)
    if gen == "sift":
        return sift(n=n, d=d, split=split, **kw)
    if gen == "large":
        return large_host(n=n, d=d, split=split, **kw)
    raise ValueError(gen)
