"""Parallel evaluation of the oracle's routed-expert FFNs for full-size sampled
checks: each worker regenerates an expert's seeded fp32 weights, encodes them
with the oracle's quantizer, decodes them and runs the fp64 FFN on the given
token rows.  Pure host code; nothing comes from the HIP library."""
import multiprocessing as mp
import os

import numpy as np

from oracle import moe, q2, q4
from synth import workloads as W


def _init_worker():
    # one BLAS / OpenMP thread per worker process
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _expert_ffn(args):
    name, layer, e, rows = args[:4]
    act = args[4] if len(args) > 4 else "exact"
    wl = W.WORKLOADS[name]
    gu4, dn4 = wl.q4_at(layer)
    codecs = (q4 if gu4 else q2, q4 if gu4 else q2, q4 if dn4 else q2)
    raw = [codecs[m].encode_matrix(W.expert_f32(wl, layer, e, m)) for m in range(3)]
    wg, wu, wd = moe.expert_weights(*raw, wl.hidden, wl.inter)
    return moe.ffn(rows, wg, wu, wd, act=act)


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

    def ffn_map(self, name, layer, act="exact"):
        def run(items):
            print("  [oracle pool] layer %d: %d expert FFNs" % (layer, len(items)), flush=True)
            return self._pool.map(_expert_ffn, [(name, layer, e, rows, act) for e, rows in items], chunksize=1)
        return run

    def close(self):
        self._pool.close()
        self._pool.join()


def layer_outputs(pool, name, jobs, topk, hidden, inter, act="exact"):
    """Oracle outputs of several layers of workload `name` for given token rows.

    jobs: list of (layer, host_layer, x_rows).  The routed FFNs of every job are
    evaluated in one parallel map (each (layer, expert) once, on the rows routed to
    it), then each layer is assembled by the oracle's own moe.layer from those
    results.  Returns a list of (out [n, H] fp64, routing dict)."""
    tasks, where = [], {}
    for l, hl, x in jobs:
        idx, _, _, _ = moe.route(x, hl.router_w, hl.router_b, topk)
        for e in np.unique(idx):
            toks, _ = np.nonzero(idx == e)           # the rows moe.layer hands to the FFN
            where[(l, int(e))] = len(tasks)
            tasks.append((name, l, int(e), np.asarray(x, np.float64)[toks], act))
    print("  [oracle pool] %d expert FFNs over %d layer job(s)" % (len(tasks), len(jobs)), flush=True)
    ys = []
    for i, y in enumerate(pool._pool.imap(_expert_ffn, tasks, chunksize=1)):
        ys.append(y)
        if (i + 1) % 64 == 0 or i + 1 == len(tasks):
            print("  [oracle pool] %d / %d expert FFNs done" % (i + 1, len(tasks)), flush=True)
    out = []
    for l, hl, x in jobs:
        def lookup(items, l=l):
            res = []
            for e, rows in items:
                i = where[(l, int(e))]
                assert np.array_equal(tasks[i][3], np.asarray(rows, np.float64))
                res.append(ys[i])
            return res
        out.append(moe.layer(x, hl.router_w, hl.router_b, None, hl.shared, topk, hidden, inter,
                             ffn_map=lookup, act=act))
    return out
