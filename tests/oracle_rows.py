"""Oracle rows of a named workload, computed in worker processes.

The FP64 oracle takes about 0.2 s per row at S = 131,072 (each row runs over
all of its keys), so the GPU tests hand large row samples to this module,
which runs as its own process (``python -m tests.oracle_rows``): it never
touches the GPU, regenerates the seeded workload, converts it to FP64 once and
forks workers that share those arrays copy-on-write, each calling the
unchanged oracle on a slice of the rows. The result is written to a .npy file.
"""

from __future__ import annotations

import argparse
import multiprocessing as mp
import os
import subprocess
import sys
import tempfile

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_SHARED = {}


def _work(groups):
    from threadpoolctl import threadpool_limits

    from oracle import flint_attention

    # one call per group of neighbouring rows: a call covers the keys up to its
    # largest row only
    with threadpool_limits(limits=1):
        return [flint_attention(rows=g, **_SHARED) for g in groups]


def compute(name: str, layer_index: int, rows: np.ndarray, workers: int) -> np.ndarray:
    from workload import make_workload

    from .common import f64, i64

    wl = make_workload(name)
    layer = wl.layers[layer_index]
    _SHARED.update(q=f64(wl.q), k=f64(wl.k), v=f64(wl.v), q_norm_w=f64(wl.q_norm_w),
                   k_norm_w=f64(wl.k_norm_w), sinks=f64(wl.sinks), cu_seqlens=i64(wl.cu_seqlens),
                   seqused=i64(wl.seqused), positions=i64(wl.positions), window=layer.window,
                   use_rope=layer.use_rope, theta=layer.theta, eps=layer.eps)
    del wl
    # groups of 4 neighbouring rows (in sorted order), dealt round-robin so
    # that every worker gets short and long rows alike
    order = np.argsort(rows, kind="stable")
    groups = [order[i:i + 4] for i in range(0, len(order), 4)]
    parts = [groups[i::workers] for i in range(workers)]
    with mp.get_context("fork").Pool(workers) as pool:
        outs = pool.map(_work, [[rows[g] for g in p] for p in parts])
    res = np.zeros((len(rows), 32, 128), np.float64)
    for p, o in zip(parts, outs):
        for g, og in zip(p, o):
            res[g] = og
    return res


def oracle_rows(name: str, layer_index: int, rows, workers: int = 8, timeout: float = 900.0):
    """Runs ``compute`` in a fresh interpreter and returns [len(rows), 32, 128]."""
    rows = np.asarray(rows, np.int64)
    with tempfile.TemporaryDirectory() as d:
        rin, rout = os.path.join(d, "rows.npy"), os.path.join(d, "out.npy")
        np.save(rin, rows)
        env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
        subprocess.run([sys.executable, "-m", "tests.oracle_rows", name, str(layer_index), rin, rout,
                        str(workers)], cwd=ROOT, env=env, check=True, timeout=timeout)
        return np.load(rout)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("name")
    ap.add_argument("layer_index", type=int)
    ap.add_argument("rows")
    ap.add_argument("out")
    ap.add_argument("workers", type=int)
    a = ap.parse_args()
    rows = np.load(a.rows)
    np.save(a.out, compute(a.name, a.layer_index, rows, a.workers))


if __name__ == "__main__":
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    main()
