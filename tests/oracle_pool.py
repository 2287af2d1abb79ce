"""The float64 oracle on whole batches, spread over worker processes.

Parity on the full-size workloads compares every output with the oracle;
with several new tokens per sequence that is many decode passes, so the
sequences are shared out to fresh interpreter processes (spawn: they never
touch the GPU). The cache arrays go to read-only memory-mapped files that
every worker maps, so they are not copied per process. Each worker calls
the oracle unchanged on its sequences.
"""

from __future__ import annotations

import os
import shutil
import tempfile

import numpy as np


def _worker(task):
    import oracle

    paths, shape, fn, q, tables, lens, scale, seqs = task
    kc = np.memmap(paths[0], dtype=np.uint16, mode="r", shape=shape)
    vc = np.memmap(paths[1], dtype=np.uint16, mode="r", shape=shape)
    f = getattr(oracle, fn)
    return seqs, f(q[seqs], kc, vc, tables[seqs], lens[seqs], scale)


def procs_available() -> int:
    n = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        n = min(n, int(os.environ["OMP_NUM_THREADS"]))
    return max(1, min(n, 16))


def oracle_batch(fn: str, q, k_cache, v_cache, block_tables, context_lens, scale, procs: int | None = None):
    """oracle.<fn>(q, k_cache, v_cache, block_tables, context_lens, scale)
    for the whole batch, the sequences split over `procs` workers."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    procs = procs or procs_available()
    S = q.shape[0]
    if procs == 1 or S < 2:
        import oracle
        return getattr(oracle, fn)(q, k_cache, v_cache, block_tables, context_lens, scale)
    tmp = tempfile.mkdtemp(prefix="pa_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    paths = (os.path.join(tmp, "k"), os.path.join(tmp, "v"))
    try:
        np.ascontiguousarray(k_cache).tofile(paths[0])
        np.ascontiguousarray(v_cache).tofile(paths[1])
        # interleaved shares balance long and short sequences
        parts = [np.arange(i, S, procs) for i in range(procs) if i < S]
        tasks = [(paths, k_cache.shape, fn, q, block_tables, context_lens, scale, p) for p in parts]
        out = np.zeros(q.shape, dtype=np.float64)
        ex = ProcessPoolExecutor(len(parts), mp_context=mp.get_context("spawn"))
        try:
            for seqs, res in ex.map(_worker, tasks, timeout=900):
                out[seqs] = res
        finally:
            ex.shutdown(wait=False, cancel_futures=True)
        return out
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
