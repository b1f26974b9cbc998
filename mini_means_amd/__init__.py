"""e-means on MI355X: Python binding of libemeans.so.

Argument marshalling only: every step of the training and assignment runs in
the HIP kernels of ``libemeans.so``. PyTorch provides the device memory and the
stream; there is no CPU fallback. If the library is not built, every call
raises.

    import torch, mini_means_amd as mm
    x = torch.randn(100_000, 64, device="cuda")
    out = mm.train(x, k=1024)               # 5 passes, scaling-law recipe
    labels, dists = mm.assign(x, out.centroids)
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libemeans.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "emeans.h")

MAX_PASSES = 64
F32, BF16, I8, F8, F16, U8 = 0, 1, 2, 3, 4, 5
LAWS = {"auto": 0, "throughput": 1, "quality": 2}
STATUS = {0: "OK", -1: "EINVAL", -2: "EDTYPE", -3: "ENOMEM", -4: "EHIP", -5: "ENOTDEVICE"}

c_i32, c_i64, c_dbl, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p


class Opts(ctypes.Structure):
    _fields_ = [
        ("dtype", c_i32), ("batch_law", c_i32), ("batch_size", c_i64), ("alpha0", c_dbl),
        ("unused_threshold", c_dbl), ("no_finalize", c_i32), ("profile", c_i32),
        ("stream", c_vp), ("trace_labels", c_vp), ("out_counts", c_vp), ("split_log", c_vp),
        ("split_log_cap", c_i64), ("max_steps", c_i64), ("bf16_search", c_i32),
        ("spherical", c_i32), ("lloyd", c_i32), ("slow_ema", c_dbl), ("slow_centroids", c_vp),
        ("search", c_i32), ("search_shift", c_vp), ("search_scale", c_dbl),
    ]


class Stats(ctypes.Structure):
    _fields_ = [
        ("batch_size", c_i64), ("total_steps", c_i64), ("n_splits", c_i64), ("n_logged", c_i64),
        ("dead_at_end", c_i64), ("alpha0", c_dbl), ("unused_threshold", c_dbl),
        ("law", c_i32), ("n_passes", c_i32),
        ("rows_per_pass", c_i64 * MAX_PASSES), ("steps_per_pass", c_i64 * MAX_PASSES),
        ("obj", c_dbl * MAX_PASSES), ("imbalance", c_dbl * MAX_PASSES),
        ("splits", c_i64 * MAX_PASSES),
        ("ms_total", c_dbl), ("ms_assign", c_dbl), ("ms_bucket", c_dbl), ("ms_group", c_dbl),
        ("ms_update", c_dbl),
        ("ms_revive", c_dbl), ("ms_sample", c_dbl), ("steps_run", c_i64),
        ("pass_ms", c_dbl * MAX_PASSES),
    ]


class EmeansError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load libemeans.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise EmeansError(f"{LIB_PATH} is missing: build it with "
                              "`python -m mini_means_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.emeans_recipe.argtypes = [c_i64, c_i32, c_i32, c_dbl, ctypes.POINTER(Opts),
                                    ctypes.POINTER(Stats)]
        L.emeans_train.argtypes = [c_vp, c_i64, c_i32, c_i32, c_dbl, ctypes.c_uint64, c_vp, c_vp,
                                   ctypes.POINTER(Opts), ctypes.POINTER(Stats)]
        L.emeans_assign.argtypes = [c_vp, c_i64, c_i32, c_vp, c_i32, c_vp, c_vp,
                                    ctypes.POINTER(Opts)]
        L.emeans_assign_static.argtypes = L.emeans_assign.argtypes
        L.emeans_batch_rows.argtypes = [c_i64, ctypes.c_uint64, c_i32, c_i64, c_i64, c_vp, c_vp]
        L.emeans_begin.argtypes = [c_i64, c_i32, c_i32, c_dbl, ctypes.c_uint64, c_vp,
                                   ctypes.POINTER(Opts), ctypes.POINTER(c_vp)]
        L.emeans_accumulate.argtypes = [c_vp, c_vp, c_i64, c_vp]
        L.emeans_update.argtypes = [c_vp]
        L.emeans_end_epoch.argtypes = [c_vp]
        L.emeans_finalize.argtypes = [c_vp, c_vp, ctypes.POINTER(Stats)]
        L.emeans_closing_add.argtypes = [c_vp, c_vp, c_i64, c_vp, c_vp]
        L.emeans_free.argtypes = [c_vp]
        L.emeans_free.restype = None
        L.emeans_int8_calibrate.argtypes = [c_vp, c_i64, c_i32, c_vp, ctypes.POINTER(c_dbl), c_vp]
        L.emeans_int8_encode.argtypes = [c_vp, c_i64, c_i32, c_vp, c_dbl, c_vp, c_vp]
        L.emeans_int8_decode.argtypes = [c_vp, c_i64, c_i32, c_vp, c_dbl, c_vp, c_vp]
        for f in ("emeans_fp8_calibrate", "emeans_fp8_encode", "emeans_fp8_decode"):
            getattr(L, f).argtypes = getattr(L, f.replace("fp8", "int8")).argtypes
            getattr(L, f).restype = ctypes.c_int
        L.emeans_last_error.restype = ctypes.c_char_p
        L.emeans_last_error.argtypes = []
        L.emeans_version.argtypes = []
        for f in ("emeans_recipe", "emeans_train", "emeans_assign", "emeans_assign_static",
                  "emeans_batch_rows",
                  "emeans_version", "emeans_begin", "emeans_accumulate", "emeans_update",
                  "emeans_end_epoch", "emeans_finalize", "emeans_closing_add",
                  "emeans_int8_calibrate",
                  "emeans_int8_encode", "emeans_int8_decode"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def declared_functions() -> list:
    """Function names the C header declares."""
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"^\s*(?:int|void|const char\*)\s+(emeans_\w+)\s*\(", text, flags=re.M)


def _check(rc: int) -> None:
    if rc != 0:
        msg = lib().emeans_last_error().decode(errors="replace")
        raise EmeansError(f"{STATUS.get(rc, rc)}: {msg}")


def _opts(dtype=F32, batch_law="auto", batch_size=0, alpha0=0.0, unused_threshold=None,
          finalize=True, profile=False, stream=None, lloyd=False) -> Opts:
    o = Opts()
    o.lloyd = 1 if lloyd else 0
    o.dtype = dtype
    o.batch_law = LAWS[batch_law] if isinstance(batch_law, str) else int(batch_law)
    o.batch_size = int(batch_size or 0)
    o.alpha0 = float(alpha0 or 0.0)
    # ABI: 0 = default, < 0 = off, > 0 = value; Python: None = default, 0 = off
    if unused_threshold is None:
        o.unused_threshold = 0.0
    elif unused_threshold <= 0:
        o.unused_threshold = -1.0
    else:
        o.unused_threshold = float(unused_threshold)
    o.no_finalize = 0 if finalize else 1
    o.profile = 1 if profile else 0
    o.stream = stream
    return o


SEARCH = {"bf16": BF16, "f16": F16, "fp16": F16, "f8": F8, "fp8": F8}


def _set_search(o: Opts, search, search_shift, search_scale, d: int):
    """On-the-fly search converter of fp32 data: search = 'bf16' | 'f16' |
    'f8' (None: none), search_shift = d float32 GPU tensor or None (centering
    for the casts, the FP8 converter's shift), search_scale (the FP8
    converter's power-of-two scale)."""
    if search is None:
        if search_shift is not None or search_scale is not None:
            raise EmeansError("EINVAL: search_shift / search_scale need search=")
        return
    if search not in SEARCH:
        raise EmeansError(f"EINVAL: search must be one of {sorted(SEARCH)} (got {search!r})")
    o.search = SEARCH[search]
    if search_shift is not None:
        _f32_device(search_shift, "search_shift")
        if search_shift.numel() != d:
            raise EmeansError(f"EINVAL: search_shift must have {d} values")
        o.search_shift = search_shift.data_ptr()
    o.search_scale = float(search_scale) if search_scale is not None else 0.0


def _stats_dict(s: Stats) -> dict:
    P = s.n_passes
    return dict(batch_size=s.batch_size, alpha0=s.alpha0, law=s.law, total_steps=s.total_steps,
                n_passes=P, epoch_rows=list(s.rows_per_pass[:P]),
                steps_per_pass=list(s.steps_per_pass[:P]), unused_threshold=s.unused_threshold,
                obj=list(s.obj[:P]), imbalance=list(s.imbalance[:P]), splits=list(s.splits[:P]),
                n_splits=s.n_splits, dead_at_end=s.dead_at_end, ms_total=s.ms_total,
                ms_assign=s.ms_assign, ms_bucket=s.ms_bucket, ms_group=s.ms_group,
                ms_update=s.ms_update,
                ms_revive=s.ms_revive, ms_sample=s.ms_sample, steps_run=s.steps_run,
                pass_ms=list(s.pass_ms[:P]))


def recipe(n: int, d: int, k: int, T: float = 5.0, **kw) -> dict:
    """Scaling-law recipe (host only): batch size, alpha0, passes and steps."""
    s = Stats()
    o = _opts(**kw)
    _check(lib().emeans_recipe(int(n), int(d), int(k), float(T), ctypes.byref(o), ctypes.byref(s)))
    return _stats_dict(s)


def _dtype_of(X) -> int:
    import torch
    if X.dtype == torch.float32:
        return F32
    if X.dtype == torch.bfloat16:
        return BF16
    if X.dtype == torch.int8:
        return I8
    if X.dtype == torch.float8_e4m3fn:
        return F8
    if X.dtype == torch.float16:
        return F16
    if X.dtype == torch.uint8:
        return U8
    raise EmeansError(f"EDTYPE: {X.dtype} not supported (float32, bfloat16, float16, int8, "
                      f"uint8 or float8_e4m3fn)")


def _stream_ptr(X, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(X.device)
    return ctypes.c_void_p(s.cuda_stream)


def _require_device(X) -> None:
    if not getattr(X, "is_cuda", False):
        raise EmeansError("ENOTDEVICE: X must be a tensor on the GPU")
    if not X.is_contiguous():
        raise EmeansError("EINVAL: X must be contiguous")


@dataclass
class TrainOutput:
    centroids: object          # k x d float32 tensor
    labels: object             # n int32 tensor or None
    stats: dict
    trace: object = None       # int32 tensor of every step's labels, or None
    counts: object = None      # k float32 running counts at the end, or None
    split_log: Optional[list] = None
    slow_centroids: object = None  # k x d float32 slow-EMA centroids (slow_ema), or None


def train(X, k: int, T: float = 5.0, seed: int = 1234, *, batch_law="auto", batch_size: int = 0,
          alpha0: float = 0.0, unused_threshold=None, finalize: bool = True,
          capture_labels: bool = True, trace: bool = False, counts: bool = False,
          split_log_cap: int = 0, profile: bool = False, max_steps: int = 0,
          bf16_search: bool = False, spherical: bool = False, lloyd: bool = False,
          slow_ema: float = 0.0, search=None, search_shift=None, search_scale=None,
          stream=None) -> TrainOutput:
    """e-means training of X (n x d tensor on the GPU). lloyd: Lloyd
    iterations instead (T of them, every row each time, alpha = 1; clusters
    left without rows are split off donors after every iteration but the
    last, as Faiss's k-means does).
    slow_ema = kappa >= 1: also the centroids of a second, slower EMA over the
    last pass (rate alpha_t / kappa), for unseen data (out.slow_centroids).
    search = 'bf16' | 'f16' | 'f8' with search_shift / search_scale: fp32 rows
    converted batch by batch for the search (casts with optional centering,
    or the calibrated FP8 converter); results stay in data units."""
    import torch
    _require_device(X)
    n, d = X.shape
    dev = X.device
    with torch.cuda.device(dev):
        o = _opts(_dtype_of(X), batch_law, batch_size, alpha0, unused_threshold, finalize,
                  profile, _stream_ptr(X, stream), lloyd)
        rc = recipe(n, d, k, T, batch_law=batch_law, batch_size=batch_size, alpha0=alpha0,
                    unused_threshold=unused_threshold, lloyd=lloyd)
        C = torch.empty((k, d), dtype=torch.float32, device=dev)
        labels = torch.empty((n,), dtype=torch.int32, device=dev) if capture_labels else None
        tr = torch.empty((sum(rc["epoch_rows"]),), dtype=torch.int32, device=dev) if trace else None
        cn = torch.empty((k,), dtype=torch.float32, device=dev) if counts else None
        log = (ctypes.c_int32 * (3 * split_log_cap))() if split_log_cap > 0 else None
        if tr is not None:
            o.trace_labels = tr.data_ptr()
        if cn is not None:
            o.out_counts = cn.data_ptr()
        if log is not None:
            o.split_log = ctypes.cast(log, c_vp)
            o.split_log_cap = split_log_cap
        o.max_steps = int(max_steps)
        o.bf16_search = 1 if bf16_search else 0
        o.spherical = 1 if spherical else 0
        _set_search(o, search, search_shift, search_scale, d)
        SC = None
        if slow_ema:
            SC = torch.empty((k, d), dtype=torch.float32, device=dev)
            o.slow_ema = float(slow_ema)
            o.slow_centroids = SC.data_ptr()
        s = Stats()
        _check(lib().emeans_train(X.data_ptr(), n, d, int(k), float(T), int(seed) & (2**64 - 1),
                                  C.data_ptr(), labels.data_ptr() if labels is not None else None,
                                  ctypes.byref(o), ctypes.byref(s)))
        st = _stats_dict(s)
        splits = None
        if log is not None:
            m = min(s.n_logged, split_log_cap)
            splits = [(log[3 * i], log[3 * i + 1], log[3 * i + 2]) for i in range(m)]
        return TrainOutput(C, labels, st, tr, cn, splits, SC)


def assign(X, C, *, with_dists: bool = True, bf16_search: bool = False, spherical: bool = False,
           search=None, search_shift=None, search_scale=None, stream=None, no_alloc: bool = False,
           out=None):
    """Nearest centroid (int32 labels) and squared distance (float32) of each row.
    bf16_search: search fp32 rows in bf16 (rows and centroids rounded).
    search / search_shift / search_scale: the general converter (as train).
    spherical: the centroid of largest dot product, and that similarity.
    no_alloc: call emeans_assign_static (the library allocates nothing; its
    working memory is one fixed device array per GPU, shared by every call).
    out: (labels, dists or None) tensors to write into instead of new ones."""
    import torch
    _require_device(X)
    if not (getattr(C, "is_cuda", False) and C.dtype == torch.float32 and C.is_contiguous()):
        raise EmeansError("EINVAL: C must be a contiguous float32 tensor on the GPU")
    n, d = X.shape
    k = C.shape[0]
    if C.shape[1] != d:
        raise EmeansError("EINVAL: C and X differ in dimension")
    with torch.cuda.device(X.device):
        if out is not None:
            labels, dists = out
            if not (getattr(labels, "is_cuda", False) and labels.dtype == torch.int32
                    and labels.is_contiguous() and labels.numel() >= n):
                raise EmeansError("EINVAL: out labels must be a contiguous int32 GPU tensor of n")
            if dists is not None and not (getattr(dists, "is_cuda", False)
                                          and dists.dtype == torch.float32
                                          and dists.is_contiguous() and dists.numel() >= n):
                raise EmeansError("EINVAL: out dists must be a contiguous float32 GPU tensor of n")
        else:
            labels = torch.empty((n,), dtype=torch.int32, device=X.device)
            dists = torch.empty((n,), dtype=torch.float32, device=X.device) if with_dists else None
        o = _opts(_dtype_of(X), stream=_stream_ptr(X, stream))
        o.bf16_search = 1 if bf16_search else 0
        o.spherical = 1 if spherical else 0
        _set_search(o, search, search_shift, search_scale, d)
        fn = lib().emeans_assign_static if no_alloc else lib().emeans_assign
        if n:
            _check(fn(X.data_ptr(), n, d, C.data_ptr(), k, labels.data_ptr(),
                      dists.data_ptr() if dists is not None else None, ctypes.byref(o)))
    return labels, dists


def _f32_device(A, what: str):
    import torch
    if not (getattr(A, "is_cuda", False) and A.dtype == torch.float32 and A.is_contiguous()):
        raise EmeansError(f"EINVAL: {what} must be a contiguous float32 tensor on the GPU")


def _calibrate(sample, stream, fn):
    import torch
    _require_device(sample)
    _f32_device(sample, "sample")
    n, d = sample.shape
    shift = torch.empty((d,), dtype=torch.float32, device=sample.device)
    scale = c_dbl(0.0)
    with torch.cuda.device(sample.device):
        _check(getattr(lib(), fn)(sample.data_ptr(), n, d, shift.data_ptr(), ctypes.byref(scale),
                                  _stream_ptr(sample, stream)))
    return shift, scale.value


def _encode(X, shift, scale, stream, fn, dtype):
    import torch
    _require_device(X)
    _f32_device(X, "X")
    _f32_device(shift, "shift")
    n, d = X.shape
    if shift.numel() != d:
        raise EmeansError("EINVAL: shift must have d entries")
    codes = torch.empty((n, d), dtype=dtype, device=X.device)
    with torch.cuda.device(X.device):
        _check(getattr(lib(), fn)(X.data_ptr(), n, d, shift.data_ptr(), float(scale),
                                  codes.data_ptr(), _stream_ptr(X, stream)))
    return codes


def _decode(C, shift, scale, stream, fn):
    import torch
    _f32_device(C, "C")
    _f32_device(shift, "shift")
    k, d = C.shape
    if shift.numel() != d:
        raise EmeansError("EINVAL: shift must have d entries")
    out = torch.empty_like(C)
    with torch.cuda.device(C.device):
        _check(getattr(lib(), fn)(C.data_ptr(), k, d, shift.data_ptr(), float(scale),
                                  out.data_ptr(), _stream_ptr(C, stream)))
    return out


def int8_calibrate(sample, stream=None):
    """README "Data precision", INT8: per-dimension shift (d float32 tensor)
    and power-of-two scale (float) from sample rows (n x d float32 tensor)."""
    return _calibrate(sample, stream, "emeans_int8_calibrate")


def int8_encode(X, shift, scale: float, stream=None):
    """int8 codes of X (n x d float32 tensor): clamp(rint((X - shift) * scale), +-127)."""
    import torch
    return _encode(X, shift, scale, stream, "emeans_int8_encode", torch.int8)


def int8_decode(C, shift, scale: float, stream=None):
    """Code-space centroids (k x d float32 tensor) back to data space: C / scale + shift."""
    return _decode(C, shift, scale, stream, "emeans_int8_decode")


def fp8_calibrate(sample, stream=None):
    """README "Data precision", FP8: as int8_calibrate, for the +-448 range of E4M3."""
    return _calibrate(sample, stream, "emeans_fp8_calibrate")


def fp8_encode(X, shift, scale: float, stream=None):
    """FP8 E4M3 codes of X (a float8_e4m3fn tensor): the nearest E4M3 value of
    (X - shift) * scale, saturating at +-448."""
    import torch
    return _encode(X, shift, scale, stream, "emeans_fp8_encode", torch.float8_e4m3fn)


def fp8_decode(C, shift, scale: float, stream=None):
    """Code-space centroids back to data space: C / scale + shift."""
    return _decode(C, shift, scale, stream, "emeans_fp8_decode")


def batch_rows(n: int, seed: int, pass_: int, start: int, count: int, device="cuda", stream=None):
    """Rows visited by slots [start, start+count) of a pass of a training run
    (pass_ = -1: the order whose first k entries are train()'s starting rows)."""
    import torch
    out = torch.empty((count,), dtype=torch.int32, device=device)
    with torch.cuda.device(out.device):
        s = stream if stream is not None else torch.cuda.current_stream(out.device)
        if count:
            _check(lib().emeans_batch_rows(int(n), int(seed) & (2**64 - 1), int(pass_),
                                           int(start), int(count), out.data_ptr(),
                                           ctypes.c_void_p(s.cuda_stream)))
    return out


class Stream:
    """Streaming training (README "Data too big for memory"): the step loop of
    train() with the rows supplied by the caller, for data that stays off the
    device. The model (centroids and running statistics) lives on the device
    of the start centroids. Pass e takes recipe["epoch_rows"][e] rows in
    batches of recipe["batch_size"] rows (the pass's last batch holds the
    rest); each batch goes in through one or more accumulate() calls followed
    by one update(), and end_epoch() closes the pass. finalize() returns the
    centroids; final_closing_mean() may first replace the closing statistics
    with a second look at the rows. All library work runs on `stream` (the
    current stream of the start centroids' device by default)."""

    def __init__(self, n: int, start, T: float = 5.0, seed: int = 1234, *, dtype=None,
                 batch_law="auto", batch_size: int = 0, alpha0: float = 0.0,
                 unused_threshold=None, finalize: bool = True, bf16_search: bool = False,
                 spherical: bool = False, profile: bool = False, counts: bool = False,
                 split_log_cap: int = 0, slow_ema: float = 0.0, search=None, search_shift=None,
                 search_scale=None, stream=None):
        import torch
        if not (getattr(start, "is_cuda", False) and start.dtype == torch.float32
                and start.is_contiguous() and start.dim() == 2):
            raise EmeansError("EINVAL: start must be a contiguous k x d float32 tensor on the GPU")
        self.k, self.d = start.shape
        self.n = int(n)
        self.device = start.device
        codes = {None: F32, torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8,
                 torch.float8_e4m3fn: F8, torch.float16: F16, torch.uint8: U8}
        code = codes.get(dtype, -1)
        if code < 0:
            raise EmeansError(f"EDTYPE: {dtype} not supported (float32, bfloat16, float16, int8, "
                              f"uint8 or float8_e4m3fn)")
        self.dtype = {F32: torch.float32, BF16: torch.bfloat16, I8: torch.int8,
                      F8: torch.float8_e4m3fn, F16: torch.float16, U8: torch.uint8}[code]
        self._stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        with torch.cuda.device(self.device):
            o = _opts(code, batch_law, batch_size, alpha0, unused_threshold, finalize, profile,
                      ctypes.c_void_p(self._stream.cuda_stream))
            o.bf16_search = 1 if bf16_search else 0
            o.spherical = 1 if spherical else 0
            _set_search(o, search, search_shift, search_scale, self.d)
            self._search_shift = search_shift   # read by the library until close()
            self._counts = torch.empty((self.k,), dtype=torch.float32, device=self.device) \
                if counts else None
            self._log = (ctypes.c_int32 * (3 * split_log_cap))() if split_log_cap > 0 else None
            if self._counts is not None:
                o.out_counts = self._counts.data_ptr()
            if self._log is not None:
                o.split_log = ctypes.cast(self._log, c_vp)
                o.split_log_cap = split_log_cap
            # the slow-EMA centroids (slow_ema) are written by finalize()
            self.slow_centroids = torch.empty((self.k, self.d), dtype=torch.float32,
                                              device=self.device) if slow_ema else None
            if self.slow_centroids is not None:
                o.slow_ema = float(slow_ema)
                o.slow_centroids = self.slow_centroids.data_ptr()
            self._opts = o
            self.recipe = recipe(self.n, self.d, self.k, T, batch_law=batch_law,
                                 batch_size=batch_size, alpha0=alpha0,
                                 unused_threshold=unused_threshold)
            h = c_vp()
            _check(lib().emeans_begin(self.n, self.d, self.k, float(T), int(seed) & (2**64 - 1),
                                      start.data_ptr(), ctypes.byref(o), ctypes.byref(h)))
            self._h = h
        self.stats = None

    def _handle(self):
        if self._h is None or not self._h.value:
            raise EmeansError("EINVAL: the model was closed")
        return self._h

    def accumulate(self, batch, labels: bool = True):
        """Add a batch (or a piece of one); returns its labels (int32) or None."""
        import torch
        _require_device(batch)
        if batch.dtype != self.dtype or batch.dim() != 2 or batch.shape[1] != self.d:
            raise EmeansError(f"EINVAL: batch must be rows x {self.d} {self.dtype}")
        with torch.cuda.stream(self._stream):   # allocated where the library writes it
            out = torch.empty((batch.shape[0],), dtype=torch.int32, device=self.device) \
                if labels else None
        _check(lib().emeans_accumulate(self._handle(), batch.data_ptr(), int(batch.shape[0]),
                                       out.data_ptr() if out is not None else None))
        return out

    def update(self, _accumulated=None) -> None:
        _check(lib().emeans_update(self._handle()))

    def end_epoch(self) -> None:
        _check(lib().emeans_end_epoch(self._handle()))

    def final_closing_mean(self, batches, assignments=None, labels_out: bool = False):
        """Replace the closing statistics with a second look at the rows
        (README "Several GPUs", final_closing_mean), after the last
        end_epoch() and before finalize().

        batches: device tensors (rows x d, the model's dtype, row-major) that
        together go over the rows in one fixed order. assignments: None, or
        one label per row in that same order (int32 or int64, host or device;
        -1 for a row the last pass skipped): the labels kept from the final
        pass, so that no search is needed. Without them every row is assigned
        once more against the final EMA centroids. Blocks larger than the
        batch size are sent in pieces. finalize() then gives each centroid the
        exact mean of the rows counted under it (the EMA centroid where none
        was). With labels_out, returns the labels used (int32, device, the
        concatenation over the batches)."""
        import torch
        B = int(self.recipe["batch_size"])
        lab_all = None
        if assignments is not None:
            lab_all = torch.as_tensor(assignments)
            if lab_all.dim() != 1 or lab_all.dtype not in (torch.int32, torch.int64):
                raise EmeansError("EINVAL: assignments must be one int32 or int64 label per row")
        used = []
        pos = 0
        with torch.cuda.device(self.device), torch.cuda.stream(self._stream):
            for batch in batches:
                _require_device(batch)
                if (batch.dtype != self.dtype or batch.dim() != 2 or batch.shape[1] != self.d
                        or not batch.is_contiguous()):
                    raise EmeansError(f"EINVAL: batches must be contiguous rows x {self.d} "
                                      f"{self.dtype} tensors")
                m = int(batch.shape[0])
                for a in range(0, m, B):
                    piece = batch[a:a + B]
                    nb = int(piece.shape[0])
                    lab = None
                    if lab_all is not None:
                        if pos + a + nb > lab_all.numel():
                            raise EmeansError("EINVAL: assignments hold fewer labels than the "
                                              "batches have rows")
                        lab = lab_all[pos + a:pos + a + nb].to(self.device, torch.int32)
                    out = torch.empty((nb,), dtype=torch.int32, device=self.device) \
                        if labels_out else None
                    _check(lib().emeans_closing_add(
                        self._handle(), piece.data_ptr(), nb,
                        lab.data_ptr() if lab is not None else None,
                        out.data_ptr() if out is not None else None))
                    if out is not None:
                        used.append(out)
                pos += m
        if lab_all is not None and pos != lab_all.numel():
            raise EmeansError("EINVAL: assignments hold more labels than the batches have rows")
        if labels_out:
            return torch.cat(used) if used else torch.zeros(0, dtype=torch.int32,
                                                             device=self.device)
        return None

    def finalize(self):
        """Centroids (k x d float32): the closing mean once every pass ended."""
        import torch
        C = torch.empty((self.k, self.d), dtype=torch.float32, device=self.device)
        s = Stats()
        _check(lib().emeans_finalize(self._handle(), C.data_ptr(), ctypes.byref(s)))
        self.stats = _stats_dict(s)
        return C

    @property
    def counts(self):
        return self._counts

    @property
    def split_log(self):
        if self._log is None or self.stats is None:
            return None
        m = self.stats["n_splits"] if self.stats["n_splits"] < len(self._log) // 3 else len(self._log) // 3
        return [tuple(self._log[3 * i:3 * i + 3]) for i in range(m)]

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().emeans_free(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def begin(n: int, start, T: float = 5.0, seed: int = 1234, **kw) -> Stream:
    return Stream(n, start, T, seed, **kw)


@dataclass
class HostTrainOutput:
    centroids: object          # k x d float32 tensor
    labels: object             # n int32 numpy array (last pass) or None
    stream: "Stream"
    trace: object = None       # every batch's labels in step order (int32 numpy) or None


def train_from_host(Xh, k: int, T: float = 5.0, seed: int = 1234, *, start=None,
                    labels: bool = True, trace: bool = False, order=None, device="cuda",
                    **kw) -> HostTrainOutput:
    """Train on a host array (numpy, row-major n x d float32, e.g. a memory
    map) that need not fit on the device, through a Stream model.

    Visiting order: order(e, rows) gives the host row ids of pass e; by
    default the library's own sampler (batch_rows), i.e. the very rows
    emeans_train visits with this seed. Starting centroids: `start` (k x d
    float32 on the device), by default the rows emeans_train starts from
    (batch_rows with pass -1). With both defaults a host run sees the same
    batches as train() on resident data.

    Transfer: each batch is gathered on the host into one of two pinned
    buffers, which take turns; a copy stream moves it to the device while
    the model's stream still computes on the other one. One event per buffer
    says the copy has landed, another that the model is done reading it
    (both streams keep the default priority)."""
    import numpy as np
    import torch
    Xh = np.asarray(Xh)
    if Xh.dtype != np.float32 or Xh.ndim != 2:
        raise EmeansError("EINVAL: Xh must be an n x d float32 array")
    n, d = Xh.shape
    dev = torch.device(device)
    if start is None:
        first = batch_rows(n, seed, -1, 0, k, device=dev).cpu().numpy()
        start = torch.from_numpy(np.ascontiguousarray(Xh[first])).to(dev)
    if order is None:
        def order(e, rows):
            return batch_rows(n, seed, e, 0, rows, device=dev).cpu().numpy()
    em = Stream(n, start, T, seed, **kw)
    B = int(em.recipe["batch_size"])
    passes = em.recipe["epoch_rows"]
    # (pass, host rows) of every update step, in schedule order
    steps = [(e, ids[a:a + B]) for e, rows_e in enumerate(passes)
             for ids in [np.asarray(order(e, rows_e))] for a in range(0, rows_e, B)]
    host = [torch.empty((B, d), dtype=torch.float32).pin_memory() for _ in range(2)]
    staged = [torch.empty((B, d), dtype=torch.float32, device=dev) for _ in range(2)]
    mover = torch.cuda.Stream(device=dev)
    landed = [torch.cuda.Event() for _ in range(2)]
    released = [torch.cuda.Event() for _ in range(2)]
    for ev in released:
        ev.record(em._stream)

    def send(j):
        """Gather step j's rows into buffer j % 2 and queue its upload."""
        buf = j % 2
        ids = steps[j][1]
        released[buf].synchronize()      # the model no longer reads this buffer
        np.take(Xh, ids, axis=0, out=host[buf].numpy()[:len(ids)])
        mover.wait_event(released[buf])
        with torch.cuda.stream(mover):
            staged[buf][:len(ids)].copy_(host[buf][:len(ids)], non_blocking=True)
        landed[buf].record(mover)

    final = len(passes) - 1
    kept = []                              # (pass, rows, device labels)
    if steps:
        send(0)
    for j, (e, ids) in enumerate(steps):
        buf = j % 2
        if j + 1 < len(steps):
            send(j + 1)                  # the next upload overlaps this step
        em._stream.wait_event(landed[buf])
        want = trace or (labels and e == final)
        lab = em.accumulate(staged[buf][:len(ids)], labels=want)
        released[buf].record(em._stream)
        em.update()
        if lab is not None:
            kept.append((e, ids, lab))
        if j + 1 == len(steps) or steps[j + 1][0] != e:
            em.end_epoch()
    C = em.finalize()                    # synchronises the model's stream
    out_labels = np.full(n, -1, dtype=np.int32) if labels else None
    tr = []
    for e, ids, lab in kept:
        h = lab.cpu().numpy()
        if labels and e == final:
            out_labels[ids] = h
        if trace:
            tr.append(h)
    return HostTrainOutput(C, out_labels, em, np.concatenate(tr) if trace and tr else None)
