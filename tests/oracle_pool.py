"""A process pool for the fp64 oracle's per-expert work (test infrastructure).

At the GLM-Flash sizes the oracle spends ~0.3 s per chosen expert building its
fp64 weights, so comparing every token of a 4096-token layer touches all 288
experts.  The experts are independent: oracle.moe_layer accepts a map over its
per-expert jobs, and this module supplies one that runs them in worker
processes.  Workers are started with "spawn" (a fresh interpreter that imports
only NumPy, synth and the oracle; nothing here touches the GPU) and regenerate
each expert's bytes from synth instead of receiving them.
"""
import atexit
import concurrent.futures as cf
import multiprocessing as mp
import os

import synth

_POOL = None


class SynthExpert:
    """Picklable expert source: expert e's (q13, s13, q2, s2) regenerated from synth."""

    def __init__(self, w: synth.Workload):
        self.w = w

    def __call__(self, e):
        return synth.expert_w13(self.w, e) + synth.expert_w2(self.w, e)


def _one_blas_thread():
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except Exception:
        pass


def workers() -> int:
    # at most 12: the GPU machines give a process about 16 host cores
    return max(1, min(12, (os.cpu_count() or 2) - 1))


def pool_map(fn, jobs):
    global _POOL
    jobs = list(jobs)
    if len(jobs) <= 2:
        return list(map(fn, jobs))
    if _POOL is None:
        _POOL = cf.ProcessPoolExecutor(workers(), mp_context=mp.get_context("spawn"),
                                       initializer=_one_blas_thread)
    return list(_POOL.map(fn, jobs, chunksize=1))


@atexit.register
def _shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True, cancel_futures=True)
        _POOL = None
