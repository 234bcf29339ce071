"""Run fp64 oracle calls in parallel for full-size parity checks.

A pool of worker processes (started with "spawn", so nothing of the GPU state of the test
process is inherited), each limited to one BLAS thread, evaluates oracle functions on
slices of the inputs (one (batch, head), one KV-head group, one sequence ...).  The oracle
itself is called as it stands; this module only distributes the calls.
"""

import concurrent.futures
import multiprocessing as mp
import os

import numpy as np


def pool_size():
    """Worker count: the cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _call(task):
    name, args, kwargs = task
    import oracle
    with np.errstate(all="ignore"):
        return getattr(oracle, name)(*args, **kwargs)


def run(tasks, workers=None):
    """tasks: list of (oracle function name, args, kwargs).  Returns the results in order.
    A worker that dies makes the call raise (it is not restarted)."""
    if not tasks:
        return []
    n = min(workers or pool_size(), len(tasks))
    ctx = mp.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(n, mp_context=ctx, initializer=_init) as ex:
        return list(ex.map(_call, tasks))


def f32(t):
    """A torch tensor (bf16 or fp32, any device) as a host float32 array: bf16 values are
    exact in fp32, and fp32 halves the bytes shipped to the workers."""
    import torch
    return t.detach().to("cpu", torch.float32).numpy()


def attention_per_head(q, k, v, causal, rope_base, pos=0, window=0, row_block=1024):
    """oracle.attention over every (batch, query head), one task each.  q [B,Hq,T,d],
    k, v [B,Hkv,S,d] host arrays.  Returns (out [B,Hq,T,d], lse [B,Hq,T]) in fp64."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    tasks = []
    for b in range(B):
        for h in range(Hq):
            g = h // G
            tasks.append(("attention", (q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1]),
                          dict(causal=causal, rope_base=rope_base, pos=pos, row_block=row_block, window=window)))
    res = run(tasks)
    out = np.empty((B, Hq, T, v.shape[3]))
    lse = np.empty((B, Hq, T))
    for i, (o, l) in enumerate(res):
        b, h = divmod(i, Hq)
        out[b, h] = o[0, 0]
        lse[b, h] = l[0, 0]
    return out, lse


def attention_rows_grouped(q, k, v, rows, causal, rope_base, pos=0, window=0):
    """oracle.attention_rows for rows [n, 3] of (b, h, t), one task per (batch, KV head) so
    each task rotates its keys once.  Returns (out [n, d], lse [n]) in the order of rows."""
    rows = np.asarray(rows, dtype=np.int64)
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    groups = {}
    for i, (b, h, t) in enumerate(rows):
        groups.setdefault((int(b), int(h) // G), []).append(i)
    tasks, index = [], []
    for (b, g), idx in sorted(groups.items()):
        sub = rows[idx].copy()
        sub[:, 0] = 0
        sub[:, 1] -= g * G
        tasks.append(("attention_rows", (q[b:b + 1, g * G:(g + 1) * G], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], sub),
                      dict(causal=causal, rope_base=rope_base, pos=pos, window=window)))
        index.append(idx)
    res = run(tasks)
    out = np.empty((len(rows), v.shape[3]))
    lse = np.empty(len(rows))
    for idx, (o, l) in zip(index, res):
        out[idx] = o
        lse[idx] = l
    return out, lse


def work_item_rows(B, Hq, Hkv, T, seed, rows_per_item=1, first_rows=0):
    """Rows (b, h, t) covering every work item of the prefill kernels: for each batch, KV-head
    group and 64-row query block, `rows_per_item` random rows of random query heads of the
    group; plus the first `first_rows` rows of every head."""
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    rows = set()
    for b in range(B):
        for g in range(Hkv):
            for qb in range((T + 63) // 64):
                for _ in range(rows_per_item):
                    t = qb * 64 + int(rng.integers(64))
                    if t < T:
                        rows.add((b, g * G + int(rng.integers(G)), t))
        for h in range(Hq):
            for t in range(min(first_rows, T)):
                rows.add((b, h, t))
    return np.array(sorted(rows), dtype=np.int64)
