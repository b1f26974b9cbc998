"""Write the oracle's free-run result of a workload: e-means for T passes from
seed 1234, with nothing taken from the GPU path.

The oracle trains on the workload's synthetic rows (the same generator and
data seed the GPU tests use), then measures, in fp64 by brute force:

  * the training MSE of its closing centroids over all n rows (blog "k-means
    Reads Your Data 25 Times. Two Would Do.", the MSE of the section on
    Lloyd's algorithm: mean over rows of the squared distance to the nearest
    centroid, not divided by d);
  * the held-out MSE over the workload's held-out rows;
  * the per-pass error, the revival count and the clusters still under the
    revival threshold at the end (README "Settings and results").

The GPU's free run (tests/test_gpu_freerun_full.py) is compared with these
values: final MSE within 1e-3 relative.

    python tests/golden/make_freerun_targets.py embedding [threads] [seed]

writes tests/golden/freerun_<workload>[_s<seed>].json (no suffix for 1234).
"""
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from mini_means_amd import datagen  # noqa: E402


def main(name: str, threads: int = 0, seed: int = 1234) -> None:
    W = datagen.WORKLOADS[name]
    t0 = time.time()
    X = datagen.make(W["gen"], W["n"], W["d"])
    Xh = datagen.make(W["gen"], W["heldout"], W["d"], split=1)
    print(f"[{name}] data {X.shape} held-out {Xh.shape} in {time.time() - t0:.1f}s", flush=True)
    t1 = time.time()
    res = oracle.train(X, W["k"], W["T"], seed, nthreads=threads)
    t_train = time.time() - t1
    print(f"[{name}] oracle e-means T={W['T']}: {t_train:.0f}s, obj {res.obj}", flush=True)
    train_mse = oracle.mse(X, res.centroids, nthreads=threads)
    held_mse = oracle.mse(Xh, res.centroids, nthreads=threads)
    ema_held = oracle.mse(Xh, res.ema_centroids, nthreads=threads)
    rc = res.recipe
    out = dict(workload=name, n=W["n"], d=W["d"], k=W["k"], T=W["T"], seed=seed,
               batch_size=rc["batch_size"], alpha0=rc["alpha0"],
               total_steps=rc["total_steps"],
               obj_per_pass=[float(v) for v in res.obj],
               n_splits=len(res.split_log), dead_at_end=int(res.dead_at_end),
               train_mse=train_mse, heldout_rows=W["heldout"], heldout_mse=held_mse,
               ema_heldout_mse=ema_held,
               labels_sha1=hashlib.sha1(np.ascontiguousarray(res.labels).tobytes()).hexdigest(),
               oracle_train_seconds=t_train, threads=threads or os.cpu_count(),
               cpu_seconds=time.time() - t0,
               source="oracle.train (CPU, fp64 search), written by "
                      "tests/golden/make_freerun_targets.py")
    suffix = "" if seed == 1234 else f"_s{seed}"
    path = os.path.join(HERE, f"freerun_{name}{suffix}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"[{name}] train {train_mse:.6f} held-out {held_mse:.6f} -> {path}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1], int(sys.argv[2]) if len(sys.argv) > 2 else 0,
         int(sys.argv[3]) if len(sys.argv) > 3 else 1234)
