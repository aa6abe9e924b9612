"""The oracle's block scores of many long requests at once, one process per
request (test infrastructure for the GPU parity tests at serving scale).

Each worker regenerates its request's inputs from the seeded generator
(synth.make_request_qk: the same bits as the batch the GPU ran) and runs
oracle.request_block_scores on them, so no large array crosses a process
boundary.  Workers are spawned, not forked (the parent has a HIP runtime),
with single-threaded BLAS; at most 16 at a time.
"""
from __future__ import annotations

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

_BLAS_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _request_scores(wl, r):
    import oracle
    import synth
    q, k = synth.make_request_qk(wl, r)
    N = int(wl.lengths[r])
    b, _ = oracle.request_block_scores(q, k, 0, N, wl.hq, wl.hkv, wl.d, wl.G, wl.n)
    return b


def _single_threaded_blas():
    # runs in each worker before any task, so before NumPy is first imported there
    for v in _BLAS_VARS:
        os.environ[v] = "1"


class OraclePool:
    """Submit (workload, request) jobs; collect float64 block scores."""

    def __init__(self, workers: int = 16):
        n = max(1, min(workers, os.cpu_count() or 1))
        self.ex = ProcessPoolExecutor(max_workers=n, mp_context=multiprocessing.get_context("spawn"),
                                      initializer=_single_threaded_blas)

    def submit(self, wl, requests):
        return {r: self.ex.submit(_request_scores, wl, r) for r in requests}

    def close(self):
        self.ex.shutdown(wait=True, cancel_futures=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
