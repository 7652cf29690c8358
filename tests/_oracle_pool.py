"""Runs the fp64 oracle over independent (batch, head) slices in worker
processes, so that full-size workloads can be compared on every output.

Test infrastructure only.  The workers are fresh Python processes (spawn),
each limited to one BLAS thread; they import numpy and oracle/ only and never
touch the GPU.  Float32 arrays in a job are widened to float64 in the worker
(exact for the bf16 and fp32 values the GPU receives), which halves what is
sent to it.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

_BLAS_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def workers() -> int:
    """Worker count: the host's CPUs, at most 16 (a GPU machine's share)."""
    return max(1, min(16, os.cpu_count() or 1))


def _widen(x):
    if isinstance(x, np.ndarray) and x.dtype == np.float32:
        return x.astype(np.float64)
    return x


def _call(job):
    name, args, kwargs = job
    import oracle
    args = [_widen(a) for a in args]
    kwargs = {k: _widen(v) for k, v in kwargs.items()}
    return getattr(oracle, name)(*args, **kwargs)


def oracle_map(name: str, jobs):
    """[(args, kwargs), ...] -> [oracle.<name>(*args, **kwargs), ...], in order,
    computed in worker processes."""
    jobs = list(jobs)
    if not jobs:
        return []
    saved = {k: os.environ.get(k) for k in _BLAS_ENV}
    for k in _BLAS_ENV:
        os.environ[k] = "1"  # inherited by the workers when they start
    try:
        ctx = mp.get_context("spawn")
        with cf.ProcessPoolExecutor(max_workers=min(workers(), len(jobs)), mp_context=ctx) as ex:
            return list(ex.map(_call, [(name, a, kw) for a, kw in jobs]))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
