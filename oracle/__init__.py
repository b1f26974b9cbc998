"""e-means CPU oracle (reference semantics for the GPU library).

TEST INFRASTRUCTURE ONLY. This package is the plain, slow checker that the GPU
path is compared against. It shares no code with the library: only the tests,
the package's smoke check and the benchmark's CPU-baseline leg may import it,
and the library never does.

What it computes, and where each step comes from (pages: the faiss
``contrib/e_means`` README, "e-means: outperforming k-means in one-tenth the
epochs"; the jecision.com blog "k-means Reads Your Data 25 Times. Two Would
Do."):

* recipe            README "Scaling laws" equations (1)-(3) and their
                    constraints; "Parameters" (batch_law, note on low
                    dimension), "Manual overrides", "Settings" table.
* exact assignment  blog, section on Lloyd's algorithm: a(i) = argmin_j
                    ||x_i - c_j||^2 (``emeans_ref.c``, fp64 brute force).
* EMA update        README "How the centroid updates work" and blog "four
                    things e-means changes", first item:
                    N_j <- (1-a) N_j + a n_j,  S_j <- (1-a) S_j + a s_j,
                    c_j = S_j / N_j.
* cosine schedule   blog, second item; README "How the centroid updates
                    work": a cosine takes the step from alpha0 down to
                    alpha0 / 10.
* revival           blog, third item (checked every five batches; a cluster
                    whose running count falls under a tenth of the mean is
                    refilled by splitting a big one); README "Settings"
                    (unused_threshold).
* batch order       README "Data too big for memory": fresh random order every
                    pass, batches of exactly B except the last of each pass,
                    every vector once per pass.
* finalisation      README "How the centroid updates work", last item: each
                    centroid becomes the exact mean of the points the last pass
                    assigned to it; README "Quick start": labels come from the
                    last pass.
* spherical         README "Spherical e-means": centroids kept at norm 1
                    (an all-zero one left as is), assignment by the
                    largest dot product (``emeans_ref.c``, fp64 brute force),
                    closing mean rescaled to norm 1, error = sum of
                    2 - 2 x similarity.
* precision         README "Data precision": centroids and running sums are
                    stored in fp32; the smaller format serves the search
                    alone: for bf16 data, and for fp32 data when
                    bf16_search asks for the pages' GPU default (rows and
                    centroids rounded to bf16 for the search, fp32 rows
                    grouped). INT8 and FP8 (E4M3) codes: a per-dimension
                    offset and a single power-of-two factor calibrated on a
                    sample, values beyond its range limited to the extreme
                    code (127 / 448); training runs on the codes and the search
                    compares them with the centroids rounded to codes. UINT8
                    data is searched exactly against the centroids rounded to
                    uint8 values (clamped to [0, 255]).
* Lloyd             blog, Lloyd section: assign all, move each centroid to
                    the exact mean of its points (the Lloyd-25 target).
* closing replay    README "Several GPUs", paragraph on final_closing_mean:
                    the closing mean taken after the last pass from a second
                    look at the rows, with the labels the last pass saved
                    (-1 rows left out) or, without them, a fresh assignment
                    against the final EMA centroids.
* slow EMA          blog, closing remark of the section on what e-means
                    changes: a second running average at a lower rate gives
                    centroids meant for data outside the training set, from
                    the same run. The
                    pages give no decay; read as a second pair of running
                    statistics over the last pass at the rate alpha_t / kappa.

Readings where the pages are silent (each listed in the design notes):
power-of-two rounding in log2 space; cap = largest power of two <= n/2;
N = S = 0 at start and c_j kept while N_j = 0; the cosine runs over all update
steps, endpoints included; revival mechanics (global step counter, strict <,
donors drawn one dead cluster at a time in index order with probability
proportional to N among the clusters that were alive at the check, donor
halves, +/-2^-10 hashed-sign perturbation); finalisation over the last pass,
keeping the EMA centroid where that pass gave no point; labels of rows the last
pass did not visit are -1; random streams from Philox4x64-10.

Parity unpinned: the split geometry of a revival (halving, the +/-2^-10
hashed-sign perturbation, the sequential donor draws) is a reading of "split
a busy cluster in two"; the pages fix no values for it. It is pinned
only by properties (donor frequency proportional to N, the split identities,
fewer dead clusters than without revival).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "emeans_ref.c")
_LIB = os.path.join(_HERE, "libemeans_ref.so")

STREAM_INIT = 1
STREAM_PERM = 2
STREAM_REVIVE = 3
STREAM_SIGN = 4

SPLIT_EPS = 2.0 ** -10       # relative perturbation of a split (reading)
REVIVE_EVERY = 5             # blog: checked every five batches


def build(force: bool = False) -> str:
    """Compile the C half of the oracle with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-shared", "-fPIC",
                               "-o", _LIB, _SRC])
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.ref_philox4x64.argtypes = [vp, vp, vp]
        L.ref_perm_at.argtypes = [u64, u64, u64, u64, u64]
        L.ref_perm_at.restype = i64
        L.ref_perm_range.argtypes = [u64, u64, u64, u64, u64, u64, vp]
        L.ref_assign.argtypes = [vp, ctypes.c_int, i64, vp, i32, vp, i32, vp, vp, vp, ctypes.c_int]
        L.ref_dist_to.argtypes = [vp, ctypes.c_int, i64, vp, i32, vp, vp, vp]
        L.ref_assign_ip.argtypes = [vp, ctypes.c_int, i64, vp, i32, vp, i32, vp, vp, vp,
                                    ctypes.c_int]
        L.ref_dot_to.argtypes = [vp, ctypes.c_int, i64, vp, i32, vp, vp, vp]
        L.ref_group.argtypes = [vp, ctypes.c_int, i64, vp, vp, i32, i32, vp, vp]
        f64 = ctypes.c_double
        L.emeans_ref_recipe.argtypes = [i64, i32, i32, f64, vp, vp, vp, vp, vp]
        L.emeans_ref_recipe.restype = ctypes.c_int
        L.emeans_ref_assign.argtypes = [vp, i64, i32, vp, i32, vp, vp]
        L.emeans_ref_assign.restype = ctypes.c_int
        L.emeans_ref_train.argtypes = [vp, i64, i32, i32, f64, u64, vp, vp, vp]
        L.emeans_ref_train.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------
# random streams
# ----------------------------------------------------------------------------

def philox4x64(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.array(ctr, dtype=np.uint64))
    k = np.ascontiguousarray(np.array(key, dtype=np.uint64))
    o = np.zeros(4, dtype=np.uint64)
    lib().ref_philox4x64(_p(c), _p(k), _p(o))
    return o


def perm_range(n: int, seed: int, stream: int, pass_: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.int64)
    if count:
        lib().ref_perm_range(n, seed, stream, pass_, start, count, _p(out))
    return out


def uniform01(seed: int, t: int, j: int) -> float:
    """Revival draw for dead cluster j at step t: 53 random bits in [0, 1)."""
    w = philox4x64((j, t, 0, STREAM_REVIVE), (seed, 0))
    return float(int(w[0]) >> 11) * 2.0 ** -53


def split_signs(seed: int, t: int, j: int, d: int) -> np.ndarray:
    """+1/-1 per coordinate for the split of step t that refills cluster j.

    Coordinate u takes bit (u mod 64) of word (u // 64) mod 4 of the Philox
    block with counter word 2 = u // 256; a set bit means -1."""
    nblk = (d + 255) // 256
    words = np.concatenate([philox4x64((j, t, b, STREAM_SIGN), (seed, 0)) for b in range(nblk)])
    bits = (words[:, None] >> np.arange(64, dtype=np.uint64)[None, :]) & np.uint64(1)
    bits = bits.reshape(-1)[:d]
    return np.where(bits == 1, np.float32(-1.0), np.float32(1.0)).astype(np.float32)


# ----------------------------------------------------------------------------
# recipe: scaling laws (README "Scaling laws")
# ----------------------------------------------------------------------------

LAW_THROUGHPUT = 1
LAW_QUALITY = 2


def recipe(n: int, d: int, k: int, T: float, batch_law: int = 0, batch_size: int = 0,
           alpha0: float = 0.0, unused_threshold: float = -1.0) -> dict:
    law = batch_law if batch_law in (LAW_THROUGHPUT, LAW_QUALITY) else (
        LAW_QUALITY if d <= 16 else LAW_THROUGHPUT)
    if batch_size and batch_size > 0:
        B = min(int(batch_size), n)
    else:
        c = 0.00439175 if law == LAW_QUALITY else 0.035134                   # eq. (2) / (1)
        braw = c * math.pow(k, 0.134749) * math.pow(n, 0.876473) * math.pow(T, 0.813344)
        B = 2 ** int(math.floor(math.log2(braw) + 0.5))                        # nearest power of two
        cap = 2 ** int(math.floor(math.log2(n / 2.0))) if n >= 2 else 1        # "capped at ~n/2"
        B = max(1, min(B, cap))
    if alpha0 and alpha0 > 0:
        a0 = float(alpha0)
    else:
        a0 = (0.8244 * math.pow(k, -0.4617) * math.pow(B, 0.9003) * math.pow(n, -0.4498)
              * math.pow(T, -0.1057))                                          # eq. (3)
        a0 = min(max(a0, 1e-4), 1.0)
    full = int(math.floor(T))
    rows = [n] * full
    frac_rows = int(math.floor((T - full) * n))
    if frac_rows > 0:
        rows.append(frac_rows)
    steps = [(r + B - 1) // B for r in rows]
    if unused_threshold is None or unused_threshold < 0:
        thr = 0.0 if d <= 2 else 0.1
    else:
        thr = float(unused_threshold)
    return dict(law=law, batch_size=B, alpha0=a0, epoch_rows=rows, steps_per_pass=steps,
                total_steps=sum(steps), unused_threshold=thr)


def alphas(alpha0: float, S: int) -> np.ndarray:
    """Cosine decay from alpha0 to alpha0/10 over the S update steps (fp32)."""
    out = np.empty(S, dtype=np.float32)
    for t in range(S):
        if S == 1:
            a = alpha0
        else:
            a = alpha0 * (0.1 + 0.45 * (1.0 + math.cos(math.pi * t / (S - 1))))
        out[t] = np.float32(a)
    return out


# ----------------------------------------------------------------------------
# assignment and grouping
# ----------------------------------------------------------------------------

# UINT8 data (README "Data precision": INT8 and UINT8 input numbers). Plain
# numpy uint8 already stands for E4M3 bit patterns here, so uint8 data is
# marked by a one-field structured dtype of the same bytes: U8 data is
# `raw_uint8_array.view(U8)`.
U8 = np.dtype([("u8", np.uint8)])


def _dtype_code(X: np.ndarray) -> int:
    if X.dtype == U8:             # uint8 values 0..255
        return 5
    if X.dtype == np.float32:
        return 0
    if X.dtype == np.uint16:      # bf16 bit patterns
        return 1
    if X.dtype == np.int8:        # int8 codes
        return 2
    if X.dtype == np.uint8:       # FP8 E4M3 codes (bit patterns)
        return 3
    if X.dtype == np.float16:     # IEEE binary16
        return 4
    raise TypeError(f"unsupported data type {X.dtype}")


def to_f32(X: np.ndarray) -> np.ndarray:
    if X.dtype == U8:
        return X.view(np.uint8).astype(np.float32)
    if X.dtype == np.uint16:
        return (X.astype(np.uint32) << 16).view(np.float32)
    if X.dtype == np.int8:
        return X.astype(np.float32)
    if X.dtype == np.uint8:
        return E4M3_VALUES[X]
    if X.dtype == np.float16:
        return X.astype(np.float32)
    return X


def bf16_round(C: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    b = np.ascontiguousarray(C, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def bf16_bits(X: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), as bf16 bit patterns (uint16)."""
    return (bf16_round(X).view(np.uint32) >> 16).astype(np.uint16)


def int8_round(C: np.ndarray) -> np.ndarray:
    """Centroids (code space) -> nearest int8 code (ties to even), clamped to
    [-127, 127], returned as fp32 values."""
    return np.clip(np.rint(np.asarray(C, dtype=np.float32)), -127, 127).astype(np.float32)


def u8_round(C: np.ndarray) -> np.ndarray:
    """Centroids of uint8 data -> nearest uint8 value (ties to even), clamped
    to [0, 255], returned as fp32 values: the search compares uint8 rows with
    uint8 centroids exactly, as for int8 codes."""
    return np.clip(np.rint(np.asarray(C, dtype=np.float32)), 0, 255).astype(np.float32)


def int8_calibrate(sample: np.ndarray):
    """README "Data precision", INT8: a per-dimension offset and a single
    power-of-two factor from a sample. Readings: the shift is the sample's midrange per
    dimension (fp64, stored fp32); the scale is the largest power of two that
    maps every sample value within [-127, 127] (1 for a constant sample)."""
    return _calibrate(sample, 127.0)


def _calibrate(sample: np.ndarray, bound: float):
    """Midrange shift per dimension and the largest power-of-two scale s with
    s * r <= bound, r the sample's largest distance from its shift (1 when
    r = 0)."""
    x = np.asarray(sample, dtype=np.float32)
    mn = x.min(axis=0).astype(np.float64)
    mx = x.max(axis=0).astype(np.float64)
    shift = ((mn + mx) / 2.0).astype(np.float32)
    s64 = shift.astype(np.float64)
    r = float(np.max(np.maximum(mx - s64, s64 - mn))) if x.size else 0.0
    if r <= 0.0:
        return shift, 1.0
    scale = 2.0 ** math.floor(math.log2(bound / r))
    while scale * r > bound:    # guard the floor of a rounded logarithm
        scale /= 2.0
    while scale * 2.0 * r <= bound:
        scale *= 2.0
    return shift, scale


def int8_encode(X: np.ndarray, shift: np.ndarray, scale: float) -> np.ndarray:
    """Codes: (x - shift) * scale in fp32 (the scale is a power of two, so the
    product is exact), rounded to nearest (ties to even) and clamped to
    [-127, 127] (values beyond the calibrated range go to the edge)."""
    y = (np.asarray(X, dtype=np.float32) - np.asarray(shift, dtype=np.float32)) * np.float32(scale)
    return np.clip(np.rint(y), -127, 127).astype(np.int8)


def int8_decode(C: np.ndarray, shift: np.ndarray, scale: float) -> np.ndarray:
    """Code-space vectors (centroids) back to data space: c / scale + shift."""
    return (np.asarray(C, dtype=np.float64) / scale
            + np.asarray(shift, dtype=np.float64)).astype(np.float32)


# ----------------------------------------------------------------------------
# FP8 E4M3 (OCP 8-bit floating point, the "FP8 (E4M3)" of README "Data
# precision"): sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
# exponent 0 holds the subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN;
# no infinities; the largest finite value is 448.
# ----------------------------------------------------------------------------

def _e4m3_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float32)
    for c in range(256):
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v = float("nan")
        elif e == 0:
            v = m * 2.0 ** -9
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[c] = -v if c & 0x80 else v
    return vals


E4M3_VALUES = _e4m3_table()
E4M3_MAX = 448.0


def e4m3_round(C: np.ndarray) -> np.ndarray:
    """fp32 -> nearest E4M3 value (ties to the even mantissa), saturating at
    +-448 (README "Data precision": values beyond the range go to the edge),
    returned as fp32 values. The spacing of E4M3 values is 2^-9 below 2^-6
    and 2^(E-4) in the binade [2^(E-1), 2^E)."""
    x = np.asarray(C, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, E = np.frexp(a)
    spacing = np.where(a < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, E - 4))
    q = np.rint(a / spacing) * spacing
    return np.copysign(q, x).astype(np.float32)


def e4m3_bits(V: np.ndarray) -> np.ndarray:
    """E4M3 values (as e4m3_round returns them) -> their bit patterns (uint8)."""
    v = np.asarray(V, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    m, E = np.frexp(a)
    normal = a >= 2.0 ** -6
    code = np.where(normal, ((E - 1 + 7) << 3) | np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64),
                    np.rint(a * 512.0).astype(np.int64))
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def fp8_calibrate(sample: np.ndarray):
    """README "Data precision", FP8: as int8_calibrate, with the largest
    power-of-two scale that maps the sample within [-448, 448]."""
    return _calibrate(sample, E4M3_MAX)


def fp8_encode(X: np.ndarray, shift: np.ndarray, scale: float) -> np.ndarray:
    """FP8 codes: (x - shift) * scale in fp32 (the product by a power of two is
    exact), rounded to the nearest E4M3 value (ties to even), saturating at
    +-448; returned as bit patterns (uint8)."""
    y = (np.asarray(X, dtype=np.float32) - np.asarray(shift, dtype=np.float32)) * np.float32(scale)
    return e4m3_bits(e4m3_round(y))


def fp8_decode(C: np.ndarray, shift: np.ndarray, scale: float) -> np.ndarray:
    """Code-space vectors (centroids) back to data space: c / scale + shift."""
    return int8_decode(C, shift, scale)


def f16_round(C: np.ndarray) -> np.ndarray:
    """fp32 -> nearest IEEE binary16 (ties to even; 65520 and beyond become
    infinity, as README "Data precision" says of FP16), returned as fp32
    values (numpy's conversion)."""
    with np.errstate(over="ignore"):
        return np.asarray(C, dtype=np.float32).astype(np.float16).astype(np.float32)


@dataclass
class Converter:
    """README "Data precision", fp32 data converted batch by batch: rows and
    centroids are converted to a smaller format for the nearest-centroid
    search only, v -> fmt((v - shift) * scale) in fp32 (the product by a
    power of two is exact). fmt 'bf16' or 'f16' is the cast (scale 1; a shift
    is the optional centering, the data's mean taken out before the 16-bit
    rounding); 'f8' is the calibrated FP8 converter (shift and scale from
    fp8_calibrate). Sums and centroids stay fp32 in data units, and distances
    in the converted units are divided by scale^2, so that they are reported
    in the data's own units, as the README states for converters."""
    fmt: str
    shift: Optional[np.ndarray] = None
    scale: float = 1.0

    def __post_init__(self):
        if self.fmt not in ("bf16", "f16", "f8"):
            raise ValueError(f"unknown search format {self.fmt}")
        if self.fmt == "f8" and self.shift is None:
            raise ValueError("the FP8 converter needs a shift and a scale")

    @property
    def scale2(self) -> float:
        return float(self.scale) ** 2

    def unrounded(self, A: np.ndarray) -> np.ndarray:
        """(A - shift) * scale in fp32, before rounding to the format."""
        y = np.asarray(A, dtype=np.float32)
        if self.shift is not None:
            y = y - np.asarray(self.shift, dtype=np.float32)
        return (y * np.float32(self.scale)).astype(np.float32)

    def rows(self, X: np.ndarray) -> np.ndarray:
        """The rows in the search's storage type: bf16 bits (uint16), IEEE fp16
        or E4M3 bits (uint8)."""
        y = self.unrounded(X)
        if self.fmt == "bf16":
            return bf16_bits(y)
        if self.fmt == "f16":
            with np.errstate(over="ignore"):
                return y.astype(np.float16)
        return e4m3_bits(e4m3_round(y))

    def centroids(self, C: np.ndarray) -> np.ndarray:
        """The search centroids, as fp32 values in the converted units."""
        y = self.unrounded(C)
        return {"bf16": bf16_round, "f16": f16_round, "f8": e4m3_round}[self.fmt](y)


def converter(bf16_search: bool = False, search: Optional[str] = None,
              search_shift: Optional[np.ndarray] = None,
              search_scale: float = 1.0) -> Optional[Converter]:
    """The converter of a run's options (bf16_search = the bf16 cast)."""
    if search is None and bf16_search:
        search = "bf16"
    if search is None:
        return None
    return Converter(search, search_shift, search_scale)


def search_centroids(C: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Centroids in the search format: bf16 for bf16 data, fp16 for fp16 data,
    int8 codes for int8 data, uint8 values for uint8 data, E4M3 values for FP8
    data (README "Data precision": only the search uses the smaller format),
    fp32 otherwise."""
    if X.dtype == U8:
        return u8_round(C)
    if X.dtype == np.uint16:
        return bf16_round(C)
    if X.dtype == np.int8:
        return int8_round(C)
    if X.dtype == np.uint8:
        return e4m3_round(C)
    if X.dtype == np.float16:
        return f16_round(C)
    return np.ascontiguousarray(C, dtype=np.float32)


def assign(X: np.ndarray, C: np.ndarray, rows: Optional[np.ndarray] = None, nthreads: int = 0):
    """Nearest centroid of each (selected) row: labels, best and runner-up distance (fp64).

    C is used as given (the caller converts it to the search format)."""
    X = np.ascontiguousarray(X)
    C = np.ascontiguousarray(C, dtype=np.float32)
    d = X.shape[1]
    k = C.shape[0]
    m = X.shape[0] if rows is None else len(rows)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    lab = np.empty(m, dtype=np.int32)
    d1 = np.empty(m, dtype=np.float64)
    d2 = np.empty(m, dtype=np.float64)
    if m:
        lib().ref_assign(_p(X), _dtype_code(X), m, _p(r), d, _p(C), k, _p(lab), _p(d1), _p(d2),
                         int(nthreads))
    return lab, d1, d2


def assign_ip(X: np.ndarray, C: np.ndarray, rows: Optional[np.ndarray] = None,
              nthreads: int = 0):
    """README "Spherical e-means": the centroid of largest dot product (lowest
    index on ties): labels, best and runner-up dot product (fp64)."""
    X = np.ascontiguousarray(X)
    C = np.ascontiguousarray(C, dtype=np.float32)
    d = X.shape[1]
    k = C.shape[0]
    m = X.shape[0] if rows is None else len(rows)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    lab = np.empty(m, dtype=np.int32)
    s1 = np.empty(m, dtype=np.float64)
    s2 = np.empty(m, dtype=np.float64)
    if m:
        lib().ref_assign_ip(_p(X), _dtype_code(X), m, _p(r), d, _p(C), k, _p(lab), _p(s1), _p(s2),
                            int(nthreads))
    return lab, s1, s2


def dot_to(X: np.ndarray, C: np.ndarray, labels: np.ndarray, rows: Optional[np.ndarray] = None):
    X = np.ascontiguousarray(X)
    C = np.ascontiguousarray(C, dtype=np.float32)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    m = len(labels)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty(m, dtype=np.float64)
    if m:
        lib().ref_dot_to(_p(X), _dtype_code(X), m, _p(r), X.shape[1], _p(C), _p(labels), _p(out))
    return out


def normalize(C: np.ndarray) -> np.ndarray:
    """Each row rescaled to norm 1 (norm and quotient in fp64, stored fp32); a
    zero row stays zero (README "Spherical e-means")."""
    c = np.asarray(C, dtype=np.float32).astype(np.float64)
    nrm = np.sqrt(np.sum(c * c, axis=-1, keepdims=True))
    out = np.where(nrm > 0, c / np.where(nrm > 0, nrm, 1.0), 0.0)
    return out.astype(np.float32)


def dist_to(X: np.ndarray, C: np.ndarray, labels: np.ndarray, rows: Optional[np.ndarray] = None):
    X = np.ascontiguousarray(X)
    C = np.ascontiguousarray(C, dtype=np.float32)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    m = len(labels)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty(m, dtype=np.float64)
    if m:
        lib().ref_dist_to(_p(X), _dtype_code(X), m, _p(r), X.shape[1], _p(C), _p(labels), _p(out))
    return out


def group(X: np.ndarray, rows: Optional[np.ndarray], labels: np.ndarray, k: int):
    """Per-cluster count n_j (int64) and sum s_j (fp64) of the selected rows."""
    X = np.ascontiguousarray(X)
    d = X.shape[1]
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    m = len(labels)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    sums = np.zeros((k, d), dtype=np.float64)
    counts = np.zeros(k, dtype=np.int64)
    lib().ref_group(_p(X), _dtype_code(X), m, _p(r), _p(labels), d, k, _p(sums), _p(counts))
    return counts, sums


def abi_recipe(n: int, d: int, k: int, T: float) -> dict:
    """emeans_ref_recipe: the C mirror of the library's recipe call (default
    options): batch size, alpha0, passes, total steps, revival threshold."""
    B, S = np.zeros(1, np.int64), np.zeros(1, np.int64)
    a0, thr = np.zeros(1, np.float64), np.zeros(1, np.float64)
    npass = np.zeros(1, np.int32)
    rc = lib().emeans_ref_recipe(n, d, k, T, _p(B), _p(a0), _p(npass), _p(S), _p(thr))
    if rc:
        raise ValueError("emeans_ref_recipe rejected its arguments")
    return dict(batch_size=int(B[0]), alpha0=float(a0[0]), passes=int(npass[0]),
                total_steps=int(S[0]), unused_threshold=float(thr[0]))


def abi_assign(X: np.ndarray, C: np.ndarray):
    """emeans_ref_assign: labels and fp32 squared distances of fp32 rows."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    C = np.ascontiguousarray(C, dtype=np.float32)
    lab = np.empty(len(X), np.int32)
    dist = np.empty(len(X), np.float32)
    rc = lib().emeans_ref_assign(_p(X), len(X), X.shape[1], _p(C), len(C), _p(lab), _p(dist))
    if rc:
        raise ValueError("emeans_ref_assign rejected its arguments")
    return lab, dist


def abi_train(X: np.ndarray, k: int, T: float, seed: int = 1234):
    """emeans_ref_train: the whole run in C (fp32 rows, default options):
    centroids, last-pass labels and the number of revivals."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    C = np.empty((k, X.shape[1]), np.float32)
    lab = np.empty(len(X), np.int32)
    ns = np.zeros(1, np.int64)
    rc = lib().emeans_ref_train(_p(X), len(X), X.shape[1], k, T, seed, _p(C), _p(lab), _p(ns))
    if rc:
        raise ValueError("emeans_ref_train rejected its arguments")
    return C, lab, int(ns[0])


def mse(X: np.ndarray, C: np.ndarray, nthreads: int = 0) -> float:
    """Mean over rows of the squared distance to the nearest centroid (not / d)."""
    _, d1, _ = assign(X, search_centroids(C, X), nthreads=nthreads)
    return float(d1.mean())


# ----------------------------------------------------------------------------
# training
# ----------------------------------------------------------------------------

@dataclass
class TrainResult:
    centroids: np.ndarray           # k x d fp32 (finalised unless finalize=False)
    ema_centroids: np.ndarray       # k x d fp32 before finalisation
    labels: np.ndarray              # n int32, last-pass label, -1 if not visited
    N: np.ndarray                   # k fp32 running counts at the end
    S: np.ndarray                   # k x d fp32 running sums at the end
    recipe: dict
    alphas: np.ndarray
    obj: list = field(default_factory=list)        # per pass: mean distance while moving
    split_log: list = field(default_factory=list)  # (t, dead j, donor i)
    dead_at_end: int = 0
    label_checks: list = field(default_factory=list)  # per step, lockstep validation results
    slow_centroids: Optional[np.ndarray] = None        # k x d fp32 (slow_ema > 0)
    slow_N: Optional[np.ndarray] = None                # k fp32 slow running counts


def init_rows(n: int, k: int, seed: int) -> np.ndarray:
    """k distinct starting rows: the first k entries of the init permutation."""
    return perm_range(n, seed, STREAM_INIT, 0, 0, k)


def _revive(t: int, seed: int, thr: float, N: np.ndarray, S: np.ndarray, C: np.ndarray,
            log: list, spherical: bool = False, empty_only: bool = False) -> None:
    k, d = S.shape
    if empty_only:
        th = 0.5  # Lloyd: the clusters that received no row (N holds whole row counts)
    else:
        total = float(np.sum(N.astype(np.float64)))
        th = thr * (total / k)
    dead = np.nonzero(N.astype(np.float64) < th)[0]
    if len(dead) == 0:
        return
    live = np.ones(k, dtype=bool)
    live[dead] = False
    for j in dead:
        u = uniform01(seed, t, int(j))
        w = np.where(live, N.astype(np.float64), 0.0)
        cum = np.cumsum(w)
        target = u * cum[-1]
        i = int(np.searchsorted(cum, target, side="right"))
        if i >= k or not live[i]:
            i = int(np.nonzero(live)[0][-1])
        sig = split_signs(seed, t, int(j), d)
        half = S[i] * np.float32(0.5)
        N[i] = N[i] * np.float32(0.5)
        N[j] = N[i]
        S[j] = half * (np.float32(1.0) + np.float32(SPLIT_EPS) * sig)
        S[i] = half * (np.float32(1.0) - np.float32(SPLIT_EPS) * sig)
        C[i] = (S[i].astype(np.float64) / float(N[i])).astype(np.float32)
        C[j] = (S[j].astype(np.float64) / float(N[j])).astype(np.float32)
        if spherical:
            C[i] = normalize(C[i])
            C[j] = normalize(C[j])
        log.append((t, int(j), i))


def train(X: np.ndarray, k: int, T: float, seed: int = 1234, *, batch_law: int = 0,
          batch_size: int = 0, alpha0: float = 0.0, unused_threshold: float = -1.0,
          finalize: bool = True,
          labels_for_step: Optional[Callable[[int, np.ndarray], np.ndarray]] = None,
          check_slots: Optional[Callable[[int, int], Optional[np.ndarray]]] = None,
          check_hook: Optional[Callable[[dict], None]] = None,
          nthreads: int = 0, bf16_search: bool = False,
          spherical: bool = False, slow_ema: float = 0.0, search: Optional[str] = None,
          search_shift: Optional[np.ndarray] = None,
          search_scale: float = 1.0) -> TrainResult:
    """e-means on X (n x d, fp32 or bf16 bits), step by step.

    bf16_search: fp32 data is searched in bf16 (rows and centroids rounded to
    bf16), while the grouping, the running sums and the centroids use the
    fp32 rows (README "Data precision": only the search uses the smaller
    format). search / search_shift / search_scale: the general form, a
    Converter of fp32 data ('bf16' or 'f16' with optional centering, 'f8'
    with the calibrated shift and scale); the reported error is in data
    units.

    spherical (README "Spherical e-means"): S / N of each centroid is
    rescaled to norm 1 after every change (an all-zero centroid is left as
    is), a vector is assigned where its dot product is largest, the closing
    step rescales each cluster's exact mean to norm 1, and the error summed
    over the rows is 2 - 2 x similarity. In label checks a dot product s enters as
    -2 s (the squared distance up to a per-row constant for unit centroids).

    slow_ema = kappa >= 1 (0: off), the second, slower EMA of the blog's
    section on what e-means changes ("for unseen data"). Reading: when the last
    pass begins, a second pair (N', S') starts from (N, S); every update of
    that pass applies the same recurrence to it with the rate
    beta_t = fl32(alpha_t / kappa); a revival in that pass restarts the
    (N', S') of both halves from their split values; the slow centroids are
    S' / N' (the EMA centroid where N' = 0), rescaled to norm 1 in spherical
    mode (res.slow_centroids, res.slow_N). kappa = 1 gives the EMA centroids.

    labels_for_step(t, rows) may supply the labels of step t from elsewhere
    (lockstep replay). The oracle then checks them on the slots that
    check_slots(t, B_t) names (all slots when it returns None) against its
    own fp64 assignment, hands the check to check_hook (or keeps it in
    label_checks), and adopts them.
    """
    n, d = X.shape
    rc = recipe(n, d, k, T, batch_law, batch_size, alpha0, unused_threshold)
    B = rc["batch_size"]
    S_tot = rc["total_steps"]
    al = alphas(rc["alpha0"], S_tot)
    thr = rc["unused_threshold"]
    conv = converter(bf16_search, search, search_shift, search_scale)
    if conv is not None and X.dtype != np.float32:
        raise ValueError("a search converter takes fp32 data")
    if conv is not None and spherical and (conv.shift is not None or conv.fmt == "f8"):
        raise ValueError("spherical mode takes the plain bf16 / fp16 casts only")
    Xf = conv.rows(X) if conv is not None else X  # the search reads this; grouping reads X
    unit2 = conv.scale2 if conv is not None else 1.0

    C = np.ascontiguousarray(to_f32(X[init_rows(n, k, seed)]), dtype=np.float32)
    if spherical:
        C = normalize(C)
    N = np.zeros(k, dtype=np.float32)
    S = np.zeros((k, d), dtype=np.float32)
    LN = np.zeros(k, dtype=np.int64)
    LS = np.zeros((k, d), dtype=np.float64)
    labels_out = np.full(n, -1, dtype=np.int32)
    res = TrainResult(centroids=C, ema_centroids=C, labels=labels_out, N=N, S=S, recipe=rc,
                      alphas=al)
    if slow_ema and slow_ema < 1.0:
        raise ValueError("slow_ema must be 0 (off) or >= 1")
    N2 = S2 = None

    t = 0
    n_pass = len(rc["epoch_rows"])
    for e, rows_e in enumerate(rc["epoch_rows"]):
        last = e == n_pass - 1
        obj = 0.0
        for s in range(rc["steps_per_pass"][e]):
            Bt = min(B, rows_e - s * B)
            rows = perm_range(n, seed, STREAM_PERM, e, s * B, Bt)
            Cs = conv.centroids(C) if conv is not None else search_centroids(C, Xf)
            C32 = conv.unrounded(C) if conv is not None else C.copy()
            if spherical:
                find = lambda r: (lambda l, a, b: (l, -2.0 * a, -2.0 * b))(*assign_ip(Xf, Cs, r, nthreads))
                score_of = lambda l, r: -2.0 * dot_to(Xf, Cs, l, r)
            else:
                find = lambda r: assign(Xf, Cs, r, nthreads)
                score_of = lambda l, r: dist_to(Xf, Cs, l, r)
            if labels_for_step is None:
                lab, d1, _ = find(rows)
                dist = d1
            else:
                lab = np.ascontiguousarray(labels_for_step(t, rows), dtype=np.int32)
                slots = None if check_slots is None else check_slots(t, Bt)
                sel = rows if slots is None else rows[slots]
                olab, od1, od2 = find(sel)
                glab = lab if slots is None else lab[slots]
                gd = score_of(glab, sel)
                chk = dict(t=t, slots=slots, oracle=olab, d1=od1, d2=od2, given=glab,
                           given_dist=gd, rows=sel, C=Cs, C32=C32, spherical=spherical)
                if check_hook is not None:
                    check_hook(chk)
                else:
                    res.label_checks.append(chk)
                dist = score_of(lab, rows)
            # spherical: sum of 2 - 2 x similarity (dist holds -2 x similarity)
            obj += float(np.sum(dist)) / unit2 + (2.0 * len(rows) if spherical else 0.0)
            counts, sums = group(X, rows, lab, k)
            a = al[t]
            b = np.float32(1.0) - a
            if slow_ema and last:
                if N2 is None:   # the slow pair starts from the running statistics
                    N2, S2 = N.copy(), S.copy()
                beta = np.float32(np.float64(a) / slow_ema)
                b2 = np.float32(1.0) - beta
                N2[:] = (b2 * N2) + (beta * counts.astype(np.float32))
                S2[:] = (np.float64(b2) * S2.astype(np.float64)
                         + np.float64(beta) * sums).astype(np.float32)
            # running count in fp32, fixed operation order: fl(fl(b*N) + fl(a*n))
            N[:] = (b * N) + (a * counts.astype(np.float32))
            # running sum: fp64 arithmetic, fp32 storage
            S[:] = (np.float64(b) * S.astype(np.float64) + np.float64(a) * sums).astype(np.float32)
            pos = N > 0
            C[pos] = (S[pos].astype(np.float64) / N[pos].astype(np.float64)[:, None]).astype(np.float32)
            if spherical:
                C[pos] = normalize(C[pos])
            if last:
                LN += counts
                LS += sums
                labels_out[rows] = lab
            if thr > 0 and (t + 1) % REVIVE_EVERY == 0:
                before = len(res.split_log)
                _revive(t, seed, thr, N, S, C, res.split_log, spherical)
                if N2 is not None:   # both halves restart their slow statistics
                    for _, j, i in res.split_log[before:]:
                        N2[[i, j]] = N[[i, j]]
                        S2[[i, j]] = S[[i, j]]
            t += 1
        res.obj.append(obj / rows_e)

    res.ema_centroids = C.copy()
    if slow_ema:
        CS = C.copy()
        if N2 is not None:
            pos = N2 > 0
            CS[pos] = (S2[pos].astype(np.float64)
                       / N2[pos].astype(np.float64)[:, None]).astype(np.float32)
            if spherical:
                CS[pos] = normalize(CS[pos])
        res.slow_centroids, res.slow_N = CS, N2
    if finalize:
        pos = LN > 0
        C[pos] = (LS[pos] / LN[pos].astype(np.float64)[:, None]).astype(np.float32)
        if spherical:
            C[pos] = normalize(C[pos])
    res.centroids = C
    if thr > 0:
        th = thr * float(np.sum(N.astype(np.float64))) / k
        res.dead_at_end = int(np.sum(N.astype(np.float64) < th))
    return res


def lloyd(X: np.ndarray, k: int, iters: int, seed: int = 1234, nthreads: int = 0,
          progress: Optional[Callable[[int, float], None]] = None,
          labels_for_step: Optional[Callable[[int, np.ndarray], np.ndarray]] = None,
          check_hook: Optional[Callable[[dict], None]] = None, split_empty: bool = True,
          split_log: Optional[list] = None):
    """Lloyd's algorithm from the same k starting rows (blog, Lloyd section,
    run as Faiss's k-means): assign all rows, move each centroid to the exact
    mean of its rows. After every update but the last, each centroid that
    received no row is split off a donor, as Faiss does with empty clusters:
    the revival step of train with the dead set {j : n_j = 0} and the step
    number i of the iteration, on N = the row counts and S = the row sums in
    fp32 (donors drawn one by one in index order, in proportion to N; each
    donor's count and sum halved between the two, the halves perturbed by
    -/+ 2^-10 per coordinate). The last update's means are the result; a
    centroid that never received a row keeps its value. split_empty=False
    gives plain Lloyd (a centroid with no row stays where it is); split_log
    receives (iteration, empty cluster, donor).
    Returns the centroids after `iters` updates and the MSE seen at each assign.

    labels_for_step(i, None) may supply the labels of iteration i from
    elsewhere (lockstep replay, as in train): they are handed to check_hook
    with the oracle's own assignment and then adopted; the MSE is that of the
    adopted labels."""
    n, d = X.shape
    C = np.ascontiguousarray(to_f32(X[init_rows(n, k, seed)]), dtype=np.float32)
    hist = []
    for i in range(iters):
        Cs = search_centroids(C, X)
        lab, d1, d2 = assign(X, Cs, nthreads=nthreads)
        if labels_for_step is not None:
            given = np.asarray(labels_for_step(i, None), dtype=np.int32)
            gd = dist_to(X, Cs, given)
            if check_hook is not None:
                check_hook(dict(t=i, rows=None, C=Cs, C32=C.copy(), given=given, oracle=lab,
                                d1=d1, d2=d2, given_dist=gd))
            lab, d1 = given, gd
        hist.append(float(d1.mean()))
        if progress is not None:
            progress(len(hist), hist[-1])
        counts, sums = group(X, None, lab, k)
        pos = counts > 0
        C[pos] = (sums[pos] / counts[pos].astype(np.float64)[:, None]).astype(np.float32)
        if split_empty and i < iters - 1 and not np.all(pos):
            N = counts.astype(np.float32)
            S = sums.astype(np.float32)
            _revive(i, seed, 0.0, N, S, C, split_log if split_log is not None else [],
                    empty_only=True)
    return C, hist


def final_closing_mean(batches, C_ema: np.ndarray, assignments: Optional[np.ndarray] = None,
                       spherical: bool = False, nthreads: int = 0):
    """The closing mean taken from a second look at the rows after the last
    pass (README "Several GPUs", the paragraph on final_closing_mean for
    callers who write their own batch loop).

    `batches` is a sequence of row blocks that together go over the rows in
    one fixed order. `assignments`, when given, holds one label per row in
    that same order: the cluster the last pass gave it, or -1 for a row that
    pass did not visit (such rows are left out). Without it, every row is
    assigned once more to its nearest centroid among C_ema, the final EMA
    centroids, compared in the data's search format (highest dot product when
    spherical). Each centroid that receives at least one row becomes the exact
    mean of its rows (fp64 sums, stored fp32; rescaled to norm 1 when
    spherical); a centroid that receives none keeps its C_ema value.

    Returns (centroids, labels): the k x d fp32 result and the label each row
    was counted under (int32, -1 for rows left out)."""
    C_ema = np.ascontiguousarray(C_ema, dtype=np.float32)
    k, d = C_ema.shape
    counts = np.zeros(k, dtype=np.int64)
    sums = np.zeros((k, d), dtype=np.float64)
    used = []
    pos = 0
    for X in batches:
        X = np.ascontiguousarray(X)
        m = X.shape[0]
        if assignments is not None:
            lab = np.asarray(assignments[pos:pos + m], dtype=np.int64)
            if len(lab) != m:
                raise ValueError("assignments hold fewer labels than the batches have rows")
            if np.any((lab < -1) | (lab >= k)):
                raise ValueError("labels must be -1 or in [0, k)")
        elif spherical:
            lab = assign_ip(X, search_centroids(C_ema, X), nthreads=nthreads)[0].astype(np.int64)
        else:
            lab = assign(X, search_centroids(C_ema, X), nthreads=nthreads)[0].astype(np.int64)
        keep = np.nonzero(lab >= 0)[0]
        c, s = group(X, keep, lab[keep].astype(np.int32), k)
        counts += c
        sums += s
        used.append(lab.astype(np.int32))
        pos += m
    if assignments is not None and pos != len(assignments):
        raise ValueError("assignments hold more labels than the batches have rows")
    C = C_ema.copy()
    have = counts > 0
    C[have] = (sums[have] / counts[have].astype(np.float64)[:, None]).astype(np.float32)
    if spherical:
        C[have] = normalize(C[have])
    return C, (np.concatenate(used) if used else np.zeros(0, dtype=np.int32))


def rel_gap(X: np.ndarray, C: np.ndarray, rows: Optional[np.ndarray], labels: np.ndarray,
            d1: np.ndarray, d2: np.ndarray) -> np.ndarray:
    """(runner-up - best) / (||x||^2 + ||c_best||^2): how decided each label is,
    relative to the size of the quantities the distance is computed from."""
    Xf = to_f32(X if rows is None else X[rows]).astype(np.float64)
    xn = np.einsum("ij,ij->i", Xf, Xf)
    Cb = C[labels].astype(np.float64)
    cn = np.einsum("ij,ij->i", Cb, Cb)
    return (d2 - d1) / np.maximum(xn + cn, 1e-300)
