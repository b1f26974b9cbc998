"""Helpers for the GPU-vs-oracle parity tests.

Tolerances (the parity bar):
  * labels: equal to the oracle's wherever the oracle's runner-up gap
    (d2 - d1) exceeds 1e-5 relative to |x|^2 + |c_best|^2, the size of the
    quantities a distance is computed from; elsewhere the label must be one
    of the near-tied centroids (its distance within that band of the best).
    During low-precision training the band also covers coordinates of the
    running centroids that sit on a rounding boundary of the search format
    (bf16_flip_bound and its int8, E4M3 and fp16 analogues);
  * distances: within 1e-5 * (|x|^2 + |c|^2) of the oracle's fp64 distance
    to the same centroid;
  * centroids: relative L2 error 1e-4 (fp32 data) or 1e-2 (bf16 data);
  * running counts: bit-exact given the same labels;
  * final MSE: 1e-3 relative.
"""
from __future__ import annotations

import numpy as np

import oracle

GAP_TOL = 1e-5
DIST_TOL = 1e-5
# FP8 E4M3 data: single products are exact, but the matrix unit sums them
# with about 13 bits (measured: at most 1.6e-4 of sum |x_i q_i| for d = 32 to
# 2048 in training; at most 2.0e-4 over 128-term dot products of random E4M3
# operands, for both the 16x16x32 and the 16x16x128 FP8 instructions). A
# distance then errs by at most 2 e sum |x_i q_i| <= e (|x|^2 + |q|^2); the
# band and the distance tolerance take 5e-4, 2.5 times the largest measured e.
F8_TOL = 5e-4


# search formats whose centroids are the running centroids rounded (the
# band then covers coordinates on a rounding boundary): bf16 bits, int8
# codes, E4M3 bits, fp16, uint8 data
LOW_PRECISION = (np.uint16, np.int8, np.uint8, np.float16, oracle.U8)


def _tol(X, base):
    return F8_TOL if X.dtype == np.uint8 else base


def obj_atol(X) -> float:
    """Absolute tolerance of a mean distance (stats obj): 0 except for FP8
    data, where each distance may err by F8_TOL (|x|^2 + |q|^2); with |q|^2
    at most twice |x|^2 on average that is F8_TOL * 3 * mean |x|^2."""
    if X.dtype != np.uint8:
        return 0.0
    Xf = oracle.to_f32(X).astype(np.float64)
    return F8_TOL * 3.0 * float(np.mean(np.einsum("ij,ij->i", Xf, Xf)))


def to_device(X: np.ndarray, device="cuda"):
    import torch
    if X.dtype == oracle.U8:       # uint8 data
        return torch.from_numpy(X.view(np.uint8)).to(device)
    if X.dtype == np.uint16:
        return torch.from_numpy(X.view(np.int16)).to(device).view(torch.bfloat16)
    if X.dtype == np.uint8:        # FP8 E4M3 bit patterns
        return torch.from_numpy(X).to(device).view(torch.float8_e4m3fn)
    return torch.from_numpy(X).to(device)


def scale_of(X, C, rows, labels):
    Xf = oracle.to_f32(X if rows is None else X[rows]).astype(np.float64)
    Cb = C[labels].astype(np.float64)
    return np.einsum("ij,ij->i", Xf, Xf) + np.einsum("ij,ij->i", Cb, Cb)


def bf16_flip_bound(X, rows, C32, labels, rel=1e-5, dot=False):
    """Bound on how much a label's squared distance can change when the bf16
    search centroid is rounded from running centroids that two exact
    implementations hold with different fp32 summation orders.

    A coordinate whose fp32 value lies within `rel` (relative to the larger of
    its magnitude and the centroid's RMS coordinate) of a bf16 rounding
    boundary may round either way; each such coordinate can move the distance
    by at most (2|x - c| + r) r, with r the possible change of the rounded
    value (with dot, the score -2 x.c of spherical e-means: by 2|x| r).
    Coordinates away from a boundary round identically on both sides."""
    Xf = oracle.to_f32(X if rows is None else X[rows]).astype(np.float64)
    C = np.ascontiguousarray(C32[labels], dtype=np.float32)
    Cb = oracle.bf16_round(C).astype(np.float64)
    c64 = C.astype(np.float64)
    rms = np.sqrt(np.mean(c64 * c64, axis=1, keepdims=True))
    delta = rel * np.maximum(np.abs(c64), rms)
    bits = C.view(np.uint32)
    low = (bits & 0xFFFF).astype(np.int64)
    ulp32 = np.abs(np.nextafter(C, np.float32(np.inf), dtype=np.float32).astype(np.float64) - c64)
    ulp16 = ulp32 * 65536.0
    dist_to_boundary = np.abs(low - 0x8000) * ulp32
    r = np.where(dist_to_boundary <= delta, ulp16 + delta, 0.0)
    if dot:
        return np.sum(2.0 * np.abs(Xf) * r, axis=1)
    return np.sum((2.0 * np.abs(Xf - Cb) + r) * r, axis=1)


def int8_flip_bound(X, rows, C32, labels, rel=1e-5):
    """The int8 analogue of bf16_flip_bound: a running-centroid coordinate
    within `rel` (relative to the larger of its magnitude and the centroid's
    RMS coordinate) of a rounding boundary k + 1/2 inside the code range may
    round to either neighbouring code; each such coordinate can move the
    distance by at most 2|x - q| + 1."""
    Xf = oracle.to_f32(X if rows is None else X[rows]).astype(np.float64)
    c64 = np.ascontiguousarray(C32[labels], dtype=np.float32).astype(np.float64)
    q = oracle.int8_round(c64).astype(np.float64)
    rms = np.sqrt(np.mean(c64 * c64, axis=1, keepdims=True))
    delta = rel * np.maximum(np.abs(c64), rms)
    near = (np.abs(c64 - (np.floor(c64) + 0.5)) <= delta) & (np.abs(c64) < 127.5 + delta)
    return np.sum(np.where(near, 2.0 * np.abs(Xf - q) + 1.0, 0.0), axis=1)


def _round_flip_bound(X, rows, C32, labels, rnd, rel=1e-5, dot=False):
    """A running-centroid coordinate that the search format's rounding `rnd`
    maps differently at c - delta and c + delta (delta = rel x max(|c|, RMS
    coordinate)) lies near a rounding boundary and may round to either
    neighbour; each such coordinate can move the distance by at most
    (2|x - q| + r) r, with r the gap between the two candidates (with dot,
    the score -2 x.c of spherical e-means: by 2|x| r)."""
    Xf = oracle.to_f32(X if rows is None else X[rows]).astype(np.float64)
    c64 = np.ascontiguousarray(C32[labels], dtype=np.float32).astype(np.float64)
    q = rnd(c64).astype(np.float64)
    rms = np.sqrt(np.mean(c64 * c64, axis=1, keepdims=True))
    delta = rel * np.maximum(np.abs(c64), rms)
    r = np.abs(rnd(c64 + delta).astype(np.float64) - rnd(c64 - delta).astype(np.float64))
    if dot:
        return np.sum(2.0 * np.abs(Xf) * r, axis=1)
    return np.sum((2.0 * np.abs(Xf - q) + r) * r, axis=1)


def e4m3_flip_bound(X, rows, C32, labels, rel=1e-5):
    """The E4M3 analogue of bf16_flip_bound."""
    return _round_flip_bound(X, rows, C32, labels, oracle.e4m3_round, rel)


def u8_flip_bound(X, rows, C32, labels, rel=1e-5):
    """The uint8 analogue of int8_flip_bound (centroids rounded to [0, 255])."""
    return _round_flip_bound(X, rows, C32, labels, oracle.u8_round, rel)


def f16_flip_bound(X, rows, C32, labels, rel=1e-5, dot=False):
    """The fp16 analogue of bf16_flip_bound (fp16 data: the search centroids
    are the running centroids rounded to fp16)."""
    return _round_flip_bound(X, rows, C32, labels, oracle.f16_round, rel, dot)


def check_labels(X, Cs, rows, given, olab, d1, d2, given_dist=None, what="", C32=None,
                 dot=False):
    """Check labels `given` against the oracle's (olab, d1, d2) on the same rows.

    Every given label g must satisfy d(g) <= d1 + 1e-5 * (|x|^2 + |c_best|^2)
    (+ the bf16 rounding allowance when C32, the unrounded centroids behind a
    bf16 search, is passed). Where the oracle's runner-up gap exceeds that
    band this forces g to be the oracle's label: decided labels are exact.
    Spherical e-means (dot): d1, d2 and given_dist hold -2 x similarity."""
    given = np.asarray(given)
    assert np.all((given >= 0) & (given < Cs.shape[0]))
    if given_dist is None:
        given_dist = oracle.dist_to(X, Cs, given, rows)
    sc = scale_of(X, Cs, rows, olab)
    band = _tol(X, GAP_TOL) * sc
    if C32 is not None and X.dtype == np.int8:
        band = (band + int8_flip_bound(X, rows, C32, olab) + int8_flip_bound(X, rows, C32, given))
    elif C32 is not None and X.dtype == np.uint8:
        band = (band + e4m3_flip_bound(X, rows, C32, olab) + e4m3_flip_bound(X, rows, C32, given))
    elif C32 is not None and X.dtype == oracle.U8:
        band = (band + u8_flip_bound(X, rows, C32, olab) + u8_flip_bound(X, rows, C32, given))
    elif C32 is not None and X.dtype == np.float16:
        band = (band + f16_flip_bound(X, rows, C32, olab, dot=dot)
                + f16_flip_bound(X, rows, C32, given, dot=dot))
    elif C32 is not None:
        band = (band + bf16_flip_bound(X, rows, C32, olab, dot=dot)
                + bf16_flip_bound(X, rows, C32, given, dot=dot))
    ok = given_dist <= d1 + band
    bad = ~ok
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} labels outside the tie band, e.g. slot {int(np.argmax(bad))}: "
        f"gpu {given[bad][:5]} oracle {olab[bad][:5]} excess {(given_dist - d1 - band)[bad][:5]}")
    decided = (d2 - d1) > band
    assert np.array_equal(given[decided], olab[decided]), f"{what}: decided labels differ"
    return int(decided.sum()), int((~decided).sum()), int((~decided & (given != olab)).sum())


def check_dists(X, Cs, rows, labels, dists, what=""):
    ref = oracle.dist_to(X, Cs, labels, rows)
    sc = scale_of(X, Cs, rows, labels)
    err = np.abs(dists.astype(np.float64) - ref)
    assert np.all(err <= _tol(X, DIST_TOL) * sc + 1e-30), (
        f"{what}: distance error {err.max():.3e} (scale {sc[np.argmax(err)]:.3e})")
    assert np.all(dists >= 0)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def step_offsets(rc: dict) -> np.ndarray:
    B = rc["batch_size"]
    sizes = []
    for rows_e, steps in zip(rc["epoch_rows"], rc["steps_per_pass"]):
        for s in range(steps):
            sizes.append(min(B, rows_e - s * B))
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def lockstep(X: np.ndarray, out, k: int, T: float, seed: int, sample: int = 0,
             rng_seed: int = 0, progress: int = 0, full=None, **opts):
    """Replay a GPU training run in the oracle, adopting the GPU's labels after
    checking them (all slots, or `sample` random slots per step), and return
    the oracle's result and the check summary.

    full: {step: count} checks the first `count` slots of that step (every
    slot when count is None), i.e. one assign launch slot by slot."""
    trace = out.trace.cpu().numpy()
    conv = oracle.converter(opts.get("bf16_search", False), opts.get("search"),
                            opts.get("search_shift"), opts.get("search_scale", 1.0))
    Xs = conv.rows(X) if conv is not None else X  # what the search reads
    rc = oracle.recipe(X.shape[0], X.shape[1], k, T, opts.get("batch_law", 0),
                       opts.get("batch_size", 0), opts.get("alpha0", 0.0),
                       opts.get("unused_threshold", -1.0))
    offs = step_offsets(rc)
    assert offs[-1] == len(trace)
    rng = np.random.default_rng(rng_seed)
    summary = dict(decided=0, undecided=0, undecided_differ=0, steps=0)

    def labels_for_step(t, rows):
        return trace[offs[t]:offs[t + 1]]

    def check_slots(t, Bt):
        if full and t in full:
            cnt = full[t]
            if cnt is None or cnt >= Bt:
                summary["full_slots"] = summary.get("full_slots", 0) + Bt
                return None
            summary["full_slots"] = summary.get("full_slots", 0) + cnt
            return np.arange(cnt)
        if not sample or sample >= Bt:
            return None
        return np.sort(rng.choice(Bt, size=sample, replace=False))

    def hook(chk):
        dec, und, diff = check_labels(Xs, chk["C"], chk["rows"], chk["given"], chk["oracle"],
                                      chk["d1"], chk["d2"], chk["given_dist"],
                                      what=f"step {chk['t']}",
                                      C32=chk["C32"] if Xs.dtype in LOW_PRECISION else None,
                                      dot=chk.get("spherical", False))
        summary["decided"] += dec
        summary["undecided"] += und
        summary["undecided_differ"] += diff
        summary["steps"] += 1
        if progress and summary["steps"] % progress == 0:
            print(f"[lockstep] step {summary['steps']}/{len(offs) - 1}", flush=True)

    res = oracle.train(X, k, T, seed, labels_for_step=labels_for_step, check_slots=check_slots,
                       check_hook=hook, **opts)
    return res, summary
