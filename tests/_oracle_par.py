"""Runs the float64 oracle over the sequences of a batch on a thread pool
(test infrastructure, not collected by pytest).

Sequences are independent in the forward, and the gradients of a mean loss
over B sequences are the mean of the per-sequence gradients, so the full
result is assembled from one-sequence oracle calls: the oracle itself is
unchanged.  NumPy's BLAS and ufuncs release the GIL, so each worker runs with
one BLAS thread and the pool spreads the sequences over the host cores.
Results are combined in sequence order (deterministic).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

import oracle as O


def host_threads(cap=16):
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def _waves(fn, n, threads):
    """fn(0..n-1) on `threads` workers, yielded in order, one wave at a time
    (at most `threads` results alive at once)."""
    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        for w0 in range(0, n, threads):
            for r in ex.map(fn, range(w0, min(n, w0 + threads))):
                yield r


def eval_nats(cfg, ids, targets, P, threads=None):
    """Per-token nats [B*T] of the forward-only evaluation, one sequence per call."""
    threads = threads or host_threads()
    B = ids.shape[0]
    out = list(_waves(lambda b: O.model_eval_nats(cfg, ids[b:b + 1], targets[b:b + 1], P), B, threads))
    return np.concatenate(out)


def _axpy(acc, g, a):
    if g is None:
        return acc
    if acc is None:
        return a * g
    acc += a * g
    return acc


def train_step(cfg, ids, targets, P, threads=None):
    """(loss, nats [B*T], grads) of the mean loss over the whole batch, from
    the oracle's one-sequence training steps: loss and grads are the means of
    the per-sequence values."""
    threads = threads or host_threads()
    B = ids.shape[0]
    loss, nats, G = 0.0, [], None
    for l_b, n_b, g_b in _waves(lambda b: O.model_fwd_bwd(cfg, ids[b:b + 1], targets[b:b + 1], P), B, threads):
        loss += l_b / B
        nats.append(n_b)
        if G is None:
            G = {k: (None if v is None else (1.0 / B) * v) for k, v in g_b.items() if k != "blocks"}
            G["blocks"] = [{k: (None if v is None else (1.0 / B) * v) for k, v in gb.items()} for gb in g_b["blocks"]]
        else:
            for k, v in g_b.items():
                if k != "blocks":
                    G[k] = _axpy(G[k], v, 1.0 / B)
            for gb_acc, gb in zip(G["blocks"], g_b["blocks"]):
                for k, v in gb.items():
                    gb_acc[k] = _axpy(gb_acc[k], v, 1.0 / B)
    return loss, np.concatenate(nats), G
