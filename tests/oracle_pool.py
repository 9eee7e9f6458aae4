"""Test helper (not a test module): run a row-local oracle function over all
query rows of one head in a thread pool, one BLAS thread per worker (numpy
releases the GIL inside its matrix products and ufuncs).  Each row's result
depends on no other row, so the split changes nothing but the time."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def map_rows(fn, n, block=256):
    """fn(row_slice) -> tuple of arrays whose first axis is the slice's rows;
    returns the tuple of row-concatenated arrays for rows 0..n-1."""
    from threadpoolctl import threadpool_limits
    starts = list(range(0, n, block))
    with threadpool_limits(1):
        with ThreadPoolExecutor(workers()) as ex:
            parts = list(ex.map(lambda r0: fn(slice(r0, min(n, r0 + block))), starts))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(len(parts[0])))
