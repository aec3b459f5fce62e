"""The fp64 oracle over many rows at once, in worker processes (test infrastructure).

Rows of a batch are independent and the loss is their mean, so the gradient of
a batch is the weighted sum of per-row gradients (pinned by the accumulation
test of the oracle).  Large configurations run those rows in separate
processes: each worker is a fresh interpreter (spawned, never forked from a
process that holds the GPU), maps the inputs from .npy files, runs
oracle.loss_and_grads (or oracle.lmhead_ce) row by row and writes its fp64
sums, rounded to fp32 for transfer, back as .npy files.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile
import time

import numpy as np

from gpu_util import announce


def _limit_threads(n):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(n)
    except Exception:
        pass


def _rows_worker(args):
    d, names, n_head, jobs, threads, out_dir = args
    _limit_threads(threads)
    import oracle
    params = {k: np.load(os.path.join(d, k + ".npy"), mmap_mode="r") for k in names}
    x = np.load(os.path.join(d, "x.npy"))
    y = np.load(os.path.join(d, "y.npy"))
    acc, loss = None, 0.0
    for r, w in jobs:
        t0 = time.perf_counter()
        l, _, G = oracle.loss_and_grads(params, x[r:r + 1], y[r:r + 1], n_head, loss_scale=w)
        loss += w * l
        if acc is None:
            acc = G
        else:
            for k in acc:
                acc[k] += G[k]
        del G
        print(f"[oracle worker {os.getpid()}] row {r} in {time.perf_counter() - t0:.1f} s", flush=True)
    os.makedirs(out_dir, exist_ok=True)
    for k, v in acc.items():
        np.save(os.path.join(out_dir, k + ".npy"), v.astype(np.float32))
    return loss


def _progress_wait(res, label, total):
    t0 = time.time()
    while not res.ready():
        res.wait(30)
        announce(f"{label}: oracle workers still running ({time.time() - t0:.0f} s, {total} jobs)")
    return res.get()


def batch_loss_and_grads(params, x, y, n_head, weights, procs=4, threads=4, label="oracle"):
    """sum_r weights[r] * (loss, grads) of the row-mean losses of rows r of x, y.

    Returns (loss, {name: float32 array}).
    """
    tmp = tempfile.mkdtemp(prefix="oracle_pool_")
    try:
        names = list(params)
        for k in names:
            np.save(os.path.join(tmp, k + ".npy"), np.asarray(params[k], dtype=np.float32))
        np.save(os.path.join(tmp, "x.npy"), np.asarray(x, dtype=np.int64))
        np.save(os.path.join(tmp, "y.npy"), np.asarray(y, dtype=np.int64))
        jobs = [(r, float(w)) for r, w in enumerate(weights) if w != 0]
        procs = max(1, min(procs, len(jobs)))
        parts = [jobs[i::procs] for i in range(procs)]
        outs = [os.path.join(tmp, f"out{i}") for i in range(procs)]
        ctx = mp.get_context("spawn")
        with ctx.Pool(procs) as pool:
            res = pool.map_async(_rows_worker, [(tmp, names, n_head, parts[i], threads, outs[i])
                                                for i in range(procs)])
            losses = _progress_wait(res, label, len(jobs))
        G = {}
        for k in names:
            s = None
            for o in outs:
                a = np.load(os.path.join(o, k + ".npy")).astype(np.float64)
                s = a if s is None else s + a
            G[k] = s.astype(np.float32)
        return float(sum(losses)), G
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def _head_worker(args):
    d, chunks, N, threads, out_dir = args
    _limit_threads(threads)
    import oracle
    X = np.load(os.path.join(d, "X.npy"), mmap_mode="r")
    W = np.load(os.path.join(d, "W.npy"))
    y = np.load(os.path.join(d, "y.npy"))
    loss, dW = 0.0, None
    os.makedirs(out_dir, exist_ok=True)
    for a, b in chunks:
        t0 = time.perf_counter()
        # each chunk's mean loss weighted by its share of the N rows: the gradient is that of the mean over N
        l, _, dX, dWc = oracle.lmhead_ce(X[a:b], W, y[a:b], loss_scale=(b - a) / N)
        loss += l * (b - a) / N
        dW = dWc if dW is None else dW + dWc
        np.save(os.path.join(out_dir, f"dX_{a}.npy"), dX.astype(np.float32))
        del dX, dWc
        print(f"[oracle worker {os.getpid()}] rows {a}:{b} in {time.perf_counter() - t0:.1f} s", flush=True)
    np.save(os.path.join(out_dir, "dW.npy"), dW.astype(np.float32))
    return loss


def lmhead_loss_and_grads(X, W, y, chunk=4096, procs=4, threads=4):
    """oracle.lmhead_ce over row chunks: (mean loss, dX, dW) of the whole problem, fp32 arrays."""
    N = X.shape[0]
    tmp = tempfile.mkdtemp(prefix="oracle_head_")
    try:
        np.save(os.path.join(tmp, "X.npy"), np.asarray(X, dtype=np.float32))
        np.save(os.path.join(tmp, "W.npy"), np.asarray(W, dtype=np.float32))
        np.save(os.path.join(tmp, "y.npy"), np.asarray(y, dtype=np.int64))
        chunks = [(a, min(N, a + chunk)) for a in range(0, N, chunk)]
        procs = max(1, min(procs, len(chunks)))
        parts = [chunks[i::procs] for i in range(procs)]
        outs = [os.path.join(tmp, f"out{i}") for i in range(procs)]
        ctx = mp.get_context("spawn")
        with ctx.Pool(procs) as pool:
            res = pool.map_async(_head_worker, [(tmp, parts[i], N, threads, outs[i]) for i in range(procs)])
            losses = _progress_wait(res, "lmhead", len(chunks))
        dX = np.empty(X.shape, dtype=np.float32)
        dW = None
        for i, o in enumerate(outs):
            for a, b in parts[i]:
                dX[a:b] = np.load(os.path.join(o, f"dX_{a}.npy"))
            w = np.load(os.path.join(o, "dW.npy")).astype(np.float64)
            dW = w if dW is None else dW + w
        return float(sum(losses)), dX, dW.astype(np.float32)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
