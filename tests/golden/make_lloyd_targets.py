"""Write the Lloyd-25 reference loss of a workload with the CPU oracle.

Lloyd's algorithm with the Faiss default of 25 iterations (blog "k-means Reads
Your Data 25 Times", section on Lloyd's algorithm and Faiss's niter = 25),
from the same k starting rows as e-means with the same seed, splitting the
clusters an iteration leaves without rows as Faiss's k-means does (oracle.lloyd;
the splits are recorded). The result file
tests/golden/lloyd25_<workload>.json holds the training MSE after every
assignment and the held-out MSE of the final centroids; the benchmark's
time-to-target measurement reads the held-out value.

    python tests/golden/make_lloyd_targets.py embedding [threads]
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from mini_means_amd import datagen  # noqa: E402


def main(name: str, threads: int = 0, iters: int = 25, seed: int = 1234) -> None:
    W = datagen.WORKLOADS[name]
    t0 = time.time()
    X = datagen.make(W["gen"], W["n"], W["d"])
    Xh = datagen.make(W["gen"], W["heldout"], W["d"], split=1)
    print(f"[{name}] data {X.shape} held-out {Xh.shape} in {time.time() - t0:.1f}s", flush=True)

    def progress(i, m):
        print(f"[{name}] iter {i}/{iters} train mse {m:.6f} ({time.time() - t0:.0f}s)", flush=True)

    splits = []
    C, hist = oracle.lloyd(X, W["k"], iters, seed, nthreads=threads, progress=progress,
                           split_log=splits)
    train_mse = oracle.mse(X, C, nthreads=threads)
    held_mse = oracle.mse(Xh, C, nthreads=threads)
    out = dict(workload=name, n=W["n"], d=W["d"], k=W["k"], iters=iters, seed=seed,
               init="first k entries of the init permutation (same as e-means)",
               train_mse_history=hist, train_mse=train_mse, heldout_rows=W["heldout"],
               heldout_mse=held_mse, empty_cluster_splits=len(splits),
               splits_per_iteration=[sum(1 for t, _, _ in splits if t == i) for i in range(iters)],
               cpu_seconds=time.time() - t0,
               threads=threads or os.cpu_count(),
               source="oracle.lloyd (CPU, fp64), written by tests/golden/make_lloyd_targets.py")
    path = os.path.join(HERE, f"lloyd25_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"[{name}] train {train_mse:.6f} held-out {held_mse:.6f} -> {path}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1], int(sys.argv[2]) if len(sys.argv) > 2 else 0)
