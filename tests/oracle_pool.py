"""A process pool for the oracle's fp64 attention in the full-size GPU
parity tests (every request and every row of the largest configurations).

The oracle is plain single-threaded NumPy; one request or one chunk of query
rows is one job. Workers are started with the "spawn" method and import only
NumPy and the oracle (never torch), and conftest starts the pool before any
test touches the GPU, so no worker is forked or exec'ed from a process that
has initialised it. The pool holds at most 16 workers (the host share of one
GPU)."""

import multiprocessing as mp
import os

import numpy as np

_POOL = None


def num_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def start() -> None:
    global _POOL
    if _POOL is None:
        _POOL = mp.get_context("spawn").Pool(num_workers())


def pool():
    start()
    return _POOL


def _attention_job(args):
    import oracle
    from oracle.attention import attention_request
    q, K, V, cached, dtype = args
    return attention_request(oracle.widen(q, dtype), oracle.widen(K, dtype), oracle.widen(V, dtype), cached)


def attention(jobs, dtype: str):
    """jobs: iterable of (q [n, HQ, D], K [S, HKV, D], V, cached) in kernel
    dtype, each one request's query rows n at absolute positions cached ..
    cached + n - 1 over its first S = cached + n keys. Yields the fp64 outputs
    in job order; the arguments are consumed lazily, a few at a time."""
    return pool().imap(_attention_job, ((q, K, V, int(c), dtype) for q, K, V, c in jobs), chunksize=1)


def extend_jobs(q, K, V, cached: int, rows_per_job: int = 256):
    """One request's extend split into jobs of query rows [t0, t1): row t sees
    keys [0, cached + t], so the job needs only the first cached + t1 keys and
    its rows sit at cached + t0 onwards. Yields (t0, t1, job)."""
    E = q.shape[0]
    for t0 in range(0, E, rows_per_job):
        t1 = min(E, t0 + rows_per_job)
        yield t0, t1, (q[t0:t1], K[:cached + t1], V[:cached + t1], cached + t0)
