"""The fp64 oracle over whole batches, spread over worker processes (test infrastructure).

Workers are started with the "spawn" method, so they never inherit a process that has touched
the GPU, and they import only numpy and the oracle.  A task is one request: its rows travel as
the stored bit patterns (bf16 as uint16, or float32) and are widened exactly in the worker.
Results come back without the per-row probability vectors (the comparison needs only the
outputs, statistics and decision margins).
"""
from __future__ import annotations

import atexit
import multiprocessing as mp
import os

import numpy as np

from oracle import spec_oracle as O

_POOL = None


def n_workers():
    """Worker count: the host's cores, at most 16 (the share of one GPU's host)."""
    return max(1, min(16, os.cpu_count() or 1))


def pool():
    global _POOL
    if _POOL is None:
        _POOL = mp.get_context("spawn").Pool(n_workers())
        atexit.register(close)
    return _POOL


def close():
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None


def _widen(a, dtype):
    if a is None:
        return None
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _strip(res):
    res.target_rows = []
    res.draft_rows = []
    return res


def _request_task(args):
    b, tl, dl, ys, dtype, sp, keys = args
    t = _widen(tl, dtype)
    d = _widen(dl, dtype)
    return b, [_strip(O.verify_request(t, d, ys, sp, seed, step, b)) for seed, step in keys]


def request_args(inp, b, sp, draft=True):
    g = int(inp.gammas[b])
    c0 = int(inp.cu_draft[b])
    tl = np.ascontiguousarray(inp.target[c0 + b:c0 + b + g + 1])
    dl = None
    if draft and inp.draft is not None and sp.temperature > 0:
        dl = np.ascontiguousarray(inp.draft[c0:c0 + g])
    ys = [int(y) for y in inp.tokens[c0:c0 + g]]
    return tl, dl, ys


def verify_requests(inp, sp, keys, requests=None, draft=True):
    """Oracle results of every listed request (all by default) for each (seed, step) in keys.

    Returns {(seed, step): {b: RequestResult}}."""
    B = len(inp.gammas)
    reqs = range(B) if requests is None else requests
    tasks = []
    for b in reqs:
        tl, dl, ys = request_args(inp, b, sp, draft)
        tasks.append((b, tl, dl, ys, inp.wl.dtype, sp, list(keys)))
    out = {k: {} for k in keys}
    for b, results in pool().imap_unordered(_request_task, tasks, chunksize=1):
        for k, r in zip(keys, results):
            out[k][b] = r
    return out


def _filtered_tokens_task(args):
    rows, dtype, sp, seed = args
    x = _widen(rows, dtype)
    rng = np.random.default_rng(seed)
    toks = np.empty(x.shape[0], dtype=np.int32)
    for i in range(x.shape[0]):
        q = O.row_distribution(x[i], sp).probs
        toks[i] = int(rng.choice(x.shape[1], p=q / q.sum()))
    return toks


def filtered_draft_tokens(inp, sp, seed):
    """Draft tokens drawn from each draft row's filtered, tempered distribution (what a draft
    model sampling from its own filtered q proposes), request by request in the workers, each
    request with its own seeded generator (seed, b)."""
    B = len(inp.gammas)
    tasks = []
    for b in range(B):
        c0, g = int(inp.cu_draft[b]), int(inp.gammas[b])
        tasks.append((np.ascontiguousarray(inp.draft[c0:c0 + g]), inp.wl.dtype, sp, [seed, b]))
    for b, toks in enumerate(pool().map(_filtered_tokens_task, tasks, chunksize=1)):
        c0 = int(inp.cu_draft[b])
        inp.tokens[c0:c0 + len(toks)] = toks
    return inp
