"""The C ABI without a GPU: the library loads, exports what the header
declares, the binding's structs match the header's layout, the host-side
recipe agrees with the oracle, and bad arguments are rejected before any
device work."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import mini_means_amd as mm
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mm.LIB_PATH):
        from mini_means_amd import build
        build.build(verbose=False)
    return mm.lib()


def test_exports_every_declared_symbol(L):
    names = mm.declared_functions()
    assert set(names) >= {"emeans_recipe", "emeans_train", "emeans_assign", "emeans_batch_rows",
                          "emeans_last_error", "emeans_version"}
    for name in names:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in names:
        assert name in exported, name
    assert L.emeans_version() == 102


def _c_layout(struct, fields):
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "emeans.h"', "int main(void){",
           f'printf("%zu\\n", sizeof({struct}));']
    for f in fields:
        src.append(f'printf("%zu\\n", offsetof({struct}, {f}));')
    src.append("return 0;}")
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "l.c")
        exe = os.path.join(td, "l")
        with open(c, "w") as fh:
            fh.write("\n".join(src))
        subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        vals = [int(v) for v in subprocess.check_output([exe]).split()]
    return vals[0], vals[1:]


@pytest.mark.parametrize("struct,cls", [("emeans_opts", mm.Opts), ("emeans_stats", mm.Stats)])
def test_struct_layout_matches_header(struct, cls):
    names = [f[0] for f in cls._fields_]
    size, offs = _c_layout(struct, names)
    assert ctypes.sizeof(cls) == size
    for name, off in zip(names, offs):
        assert getattr(cls, name).offset == off, name


CASES = [(10_000, 16, 64, 5.0), (1_000_000, 768, 4096, 5.0), (1_000_000, 96, 16384, 5.0),
         (1_000_000, 128, 16384, 5.0), (100_000_000, 128, 65536, 3.0), (1, 1, 1, 1.0),
         (2, 3, 2, 0.5), (3, 2, 1, 2.5), (1000, 2, 10, 1.0), (777, 33, 5, 7.25),
         (12345, 64, 1000, 2.5), (10**7, 1024, 10**6, 1.2)]


@pytest.mark.parametrize("n,d,k,T", CASES)
def test_recipe_matches_oracle(L, n, d, k, T):
    got = mm.recipe(n, d, k, T)
    want = oracle.recipe(n, d, k, T)
    assert got["batch_size"] == want["batch_size"]
    assert got["alpha0"] == want["alpha0"]          # same formula, same libm: bit-equal
    assert got["law"] == want["law"]
    assert got["epoch_rows"] == want["epoch_rows"]
    assert got["steps_per_pass"] == want["steps_per_pass"]
    assert got["total_steps"] == want["total_steps"]
    assert got["unused_threshold"] == want["unused_threshold"]


def test_recipe_overrides(L):
    r = mm.recipe(10**6, 64, 1024, 5, batch_size=8192)
    o = oracle.recipe(10**6, 64, 1024, 5, batch_size=8192)
    assert r["batch_size"] == 8192 and r["alpha0"] == o["alpha0"]
    r = mm.recipe(10**6, 64, 1024, 5, batch_size=8192, alpha0=0.05)
    assert r["alpha0"] == 0.05
    r = mm.recipe(10**6, 64, 1024, 5, batch_law="quality")
    assert r["batch_size"] == oracle.recipe(10**6, 64, 1024, 5, batch_law=2)["batch_size"]
    assert mm.recipe(1000, 8, 4, 1, unused_threshold=0)["unused_threshold"] == 0.0
    assert mm.recipe(1000, 8, 4, 1, unused_threshold=0.2)["unused_threshold"] == 0.2
    assert mm.recipe(1000, 2, 4, 1)["unused_threshold"] == 0.0


@pytest.mark.parametrize("args,code", [
    ((10, 4, 11, 5.0), -1),      # k > n
    ((10, 0, 2, 5.0), -1),       # d < 1
    ((10, 4, 0, 5.0), -1),       # k < 1
    ((0, 4, 1, 5.0), -1),        # n < 1
    ((10, 4, 2, 0.0), -1),       # T <= 0
    ((10, 4, 2, -1.0), -1),
    ((10, 4, 2, 65.0), -1),      # too many passes
])
def test_recipe_rejects(L, args, code):
    s = mm.Stats()
    o = mm.Opts()
    assert L.emeans_recipe(*args, ctypes.byref(o), ctypes.byref(s)) == code
    assert L.emeans_last_error()


def test_lloyd_recipe(L):
    """Lloyd mode (blog, Lloyd section): T whole iterations over all n rows,
    alpha = 1, no revival; the 2^24 batch limit does not apply."""
    r = mm.recipe(1000, 16, 10, 7, lloyd=True)
    assert (r["batch_size"], r["alpha0"], r["total_steps"], r["unused_threshold"]) == (1000, 1.0, 7, 0.0)
    assert r["epoch_rows"] == [1000] * 7 and r["steps_per_pass"] == [1] * 7
    assert mm.recipe(20_000_000, 128, 100, 3, lloyd=True)["batch_size"] == 20_000_000
    for T in (2.5, 65.0):
        with pytest.raises(mm.EmeansError, match="EINVAL"):
            mm.recipe(1000, 16, 10, T, lloyd=True)
    o = mm.Opts()
    o.lloyd = 1
    s = mm.Stats()
    # streaming training takes no Lloyd mode; the check precedes device work
    m = ctypes.c_void_p()
    assert L.emeans_begin(100, 4, 3, 2.0, 1, None, ctypes.byref(o), ctypes.byref(m)) == -1
    assert b"lloyd" in L.emeans_last_error()


def test_train_rejects_before_device_work(L):
    o = mm.Opts()
    s = mm.Stats()
    # k > n
    assert L.emeans_train(None, 10, 4, 11, 5.0, 1, None, None, ctypes.byref(o), ctypes.byref(s)) == -1
    # null pointers
    assert L.emeans_train(None, 100, 4, 3, 5.0, 1, None, None, ctypes.byref(o), ctypes.byref(s)) == -1
    assert b"NULL" in L.emeans_last_error()
    # unsupported dtype
    o.dtype = 7
    assert L.emeans_train(None, 100, 4, 3, 5.0, 1, None, None, ctypes.byref(o), ctypes.byref(s)) == -2
    o.dtype = 0
    o.batch_law = 5
    assert L.emeans_train(None, 100, 4, 3, 5.0, 1, None, None, ctypes.byref(o), ctypes.byref(s)) == -1
    o.batch_law = 0
    o.unused_threshold = 1.5
    assert L.emeans_train(None, 100, 4, 3, 5.0, 1, None, None, ctypes.byref(o), ctypes.byref(s)) == -1


def test_slow_ema_options_rejected_before_device_work(L):
    """slow_ema: kappa must be 0 or >= 1, needs an output table, and does not
    combine with Lloyd mode; the streaming begin applies the same checks."""
    s = mm.Stats()
    for kappa, table, lloyd, msg in ((0.5, 8, 0, b"slow_ema must be"),
                                     (2.0, None, 0, b"needs slow_centroids"),
                                     (0.0, 8, 0, b"slow_ema is 0"),
                                     (2.0, 8, 1, b"lloyd")):
        o = mm.Opts()
        o.slow_ema = kappa
        o.slow_centroids = table
        o.lloyd = lloyd
        assert L.emeans_train(None, 100, 4, 3, 2.0, 1, None, None, ctypes.byref(o),
                              ctypes.byref(s)) == -1
        assert msg in L.emeans_last_error()
    o = mm.Opts()
    o.slow_ema = 0.5
    h = ctypes.c_void_p()
    assert L.emeans_begin(100, 4, 3, 2.0, 1, None, ctypes.byref(o), ctypes.byref(h)) == -1
    assert b"slow_ema must be" in L.emeans_last_error()


def test_search_converter_options_rejected_before_device_work(L):
    """opts.search: a known format, fp32 data only, the FP8 converter with a
    shift and a power-of-two scale, the casts with scale 0 or 1, no centering
    or FP8 converter in spherical mode, no stray shift or scale."""
    s = mm.Stats()
    fake = 4096   # never dereferenced: the checks run before any device work
    cases = [dict(search=7), dict(search=4, dtype=1), dict(search=3),
             dict(search=3, search_shift=fake, search_scale=3.0),
             dict(search=1, search_scale=2.0), dict(search=4, bf16_search=1),
             dict(search=1, search_shift=fake, spherical=1),
             dict(search=3, search_shift=fake, search_scale=4.0, spherical=1),
             dict(search_shift=fake), dict(search_scale=8.0)]
    for c in cases:
        o = mm.Opts()
        for key, val in c.items():
            setattr(o, key, val)
        assert L.emeans_train(None, 100, 4, 3, 2.0, 1, None, None, ctypes.byref(o),
                              ctypes.byref(s)) == -1, c
        assert b"NULL" not in L.emeans_last_error()
        # assign: non-NULL pointers so that the option check is what answers
        assert L.emeans_assign(fake, 10, 4, fake, 3, fake, None, ctypes.byref(o)) == -1, c
        assert b"NULL" not in L.emeans_last_error() and b"device" not in L.emeans_last_error()


def test_assign_rejects_before_device_work(L):
    o = mm.Opts()
    assert L.emeans_assign(None, 10, 4, None, 3, None, None, ctypes.byref(o)) == -1
    assert L.emeans_assign(None, 10, 0, None, 3, None, None, ctypes.byref(o)) == -1
    assert L.emeans_assign(None, -1, 4, None, 3, None, None, ctypes.byref(o)) == -1
    o.dtype = 6   # 0..5 are fp32, bf16, int8, FP8, fp16, uint8
    assert L.emeans_assign(None, 10, 4, None, 3, None, None, ctypes.byref(o)) == -2
    assert L.emeans_batch_rows(10, 1, 0, 5, 6, None, None) == -1
    assert L.emeans_batch_rows(0, 1, 0, 0, 0, None, None) == -1


def test_static_assign_rejects_sizes_beyond_its_array(L):
    """emeans_assign_static checks its working-memory need against the fixed
    array (EMEANS_STATIC_SCRATCH_BYTES) before touching any pointer: a bf16
    search copy of k x d elements needs 2kd bytes."""
    import re
    with open(mm.HEADER) as f:
        cap = int(eval(re.search(r"#define EMEANS_STATIC_SCRATCH_BYTES \((.*)\)", f.read())
                       .group(1).replace("u", "")))
    assert cap == 32 << 20
    x = np.zeros(4, np.float32)
    o = mm.Opts()
    o.dtype = 1                      # bf16 rows: a bf16 copy of the centroids
    d = 128
    k = cap // (2 * d)               # the copy alone fills the array; the bias does not fit
    p = x.ctypes.data
    assert L.emeans_assign_static(p, 16, d, p, k, p, None, ctypes.byref(o)) == -1
    assert "scratch" in L.emeans_last_error().decode()
    # a size that fits passes the size check and reaches the pointer checks
    assert L.emeans_assign_static(p, 16, d, p, 1000, p, None, ctypes.byref(o)) == -5
    o.dtype = 0
    o.search = 4                     # the fp16 cast of fp32 rows: 2nd bytes of converted rows
    n = cap // (2 * d)
    assert L.emeans_assign_static(p, n, d, p, 8, p, None, ctypes.byref(o)) == -1
    assert L.emeans_assign_static(p, n // 2, d, p, 8, p, None, ctypes.byref(o)) == -5


def test_host_pointer_is_not_device(L):
    """A host buffer is refused with ENOTDEVICE (no GPU needed to tell)."""
    x = np.zeros((16, 4), np.float32)
    C = np.zeros((2, 4), np.float32)
    lab = np.zeros(16, np.int32)
    o = mm.Opts()
    rc = L.emeans_assign(x.ctypes.data, 16, 4, C.ctypes.data, 2, lab.ctypes.data, None,
                         ctypes.byref(o))
    assert rc == -5


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(mm.EmeansError):
        mm.train(torch.zeros(100, 4), 3)
    with pytest.raises(mm.EmeansError):
        mm.assign(torch.zeros(100, 4), torch.zeros(3, 4))
