"""Parallel evaluation of the oracle's routed-expert FFNs for full-size sampled
checks: each worker regenerates an expert's seeded fp32 weights, encodes them
with the oracle's quantizer, decodes them and runs the fp64 FFN on the given
token rows.  Pure host code; nothing comes from the HIP library."""
import multiprocessing as mp
import os

import numpy as np

from oracle import moe, q2
from synth import workloads as W


def _init_worker():
    # one BLAS / OpenMP thread per worker process
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _expert_ffn(args):
    name, layer, e, rows = args
    wl = W.WORKLOADS[name]
    raw = [q2.encode_matrix(W.expert_f32(wl, layer, e, m)) for m in range(3)]
    wg, wu, wd = moe.expert_weights(*raw, wl.hidden, wl.inter)
    return moe.ffn(rows, wg, wu, wd)


class ExpertPool:
    def __init__(self, procs=None):
        n = procs or max(1, min(16, len(os.sched_getaffinity(0))))
        # spawn, not fork: the parent may hold BLAS / HIP runtime threads
        env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
        os.environ["OMP_NUM_THREADS"] = "1"
        os.environ["OPENBLAS_NUM_THREADS"] = "1"
        try:
            self._pool = mp.get_context("spawn").Pool(n, initializer=_init_worker)
        finally:
            for k, v in env.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def ffn_map(self, name, layer):
        def run(items):
            print("  [oracle pool] layer %d: %d expert FFNs" % (layer, len(items)), flush=True)
            return self._pool.map(_expert_ffn, [(name, layer, e, rows) for e, rows in items], chunksize=1)
        return run

    def close(self):
        self._pool.close()
        self._pool.join()
