"""Evaluating the oracle over every row (or sequence) of a full-size case.

TEST INFRASTRUCTURE ONLY, like the rest of this package: used by the tests
and by the benchmark's CPU-baseline leg.

The oracle functions take the rows (prefill) or sequences (decode) to
evaluate as an argument; these helpers cut a whole case into contiguous
pieces, evaluate them in worker threads (numpy releases the interpreter lock
in its array loops and BLAS calls) and put the results back together.  Each
piece is one call of the unchanged oracle, so the values are the oracle's.
BLAS runs one thread per worker so the workers do not oversubscribe the
cores."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def _workers(n: int | None) -> int:
    if n:
        return n
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _run(fn, pieces, workers):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, pieces))


def all_rows(fn, T: int, block: int = 256, workers: int | None = None):
    """(out, lse) of fn(rows=...) over rows 0..T-1: blocks of `block` rows are
    dealt round-robin to the workers, so each gets a mix of short and long
    causal ranges."""
    workers = _workers(workers)
    blocks = [np.arange(s, min(s + block, T), dtype=np.int64) for s in range(0, T, block)]
    if not blocks:
        return fn(np.zeros(0, np.int64))
    pieces = [np.concatenate(blocks[k::workers]) for k in range(min(workers, len(blocks)))]
    res = _run(fn, pieces, len(pieces))
    out = np.empty((T,) + res[0][0].shape[1:], np.float64)
    lse = np.empty((T,) + res[0][1].shape[1:], np.float64)
    for rows, (o, ls) in zip(pieces, res):
        out[rows] = o
        lse[rows] = ls
    return out, lse


def all_batches(fn, B: int, workers: int | None = None):
    """(out, lse) of fn(batches=[...]) over sequences 0..B-1, one sequence per task."""
    workers = _workers(workers)
    res = _run(lambda b: fn([b]), list(range(B)), workers)
    return np.concatenate([o for o, _ in res]), np.concatenate([ls for _, ls in res])
