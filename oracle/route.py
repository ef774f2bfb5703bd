"""Route oracle: the batch sort of the L^3 layer (TEST INFRASTRUCTURE ONLY).

Because the layer mixes channels only, a batch can be reordered by token ID so
that tokens sharing an ID are contiguous, the layer run per ID block, and the
order undone afterwards ("L^3: Large Lookup Layers": sciencestack.ai page,
Fig. 3 caption; papernotes.org page, section "关键设计", item 3;
kimjy99.github.io page, section "2. Efficient Training and Inference").

Readings (the pages say "sort" without more): the sort is stable (ties keep
their batch order), so the permutation is unique; blocks come in ascending ID
order.  IDs outside [0, vocab) sort as the key ``vocab`` (after every valid
ID), keep their batch order, form one final block, and raise ``err``.
"""
from __future__ import annotations

import numpy as np


def _keys(ids, vocab: int) -> np.ndarray:
    ids = np.asarray(ids, dtype=np.int64)
    return np.where((ids >= 0) & (ids < vocab), ids, vocab)


def route(ids, vocab: int) -> dict:
    """Stable sort by token ID and the per-ID blocks.

    Returns int32 arrays ``perm`` (sorted position -> batch index),
    ``sorted_ids`` (the keys in sorted order), ``inv_perm`` (batch index ->
    sorted position), ``uniq`` (the distinct keys, ascending), ``counts``
    (tokens per block), ``seg_start`` (m+1 block starts, last = n), and
    ``num_segments`` (m) and ``err`` (any ID out of range)."""
    key = _keys(ids, vocab)
    n = len(key)
    perm = np.argsort(key, kind="stable")  # a stable library sort is the definition
    sk = key[perm]
    inv = np.empty(n, dtype=np.int64)
    inv[perm] = np.arange(n)
    if n:
        heads = np.flatnonzero(np.concatenate([[True], sk[1:] != sk[:-1]]))
    else:
        heads = np.zeros(0, dtype=np.int64)
    seg_start = np.concatenate([heads, [n]])
    return {
        "perm": perm.astype(np.int32),
        "sorted_ids": sk.astype(np.int32),
        "inv_perm": inv.astype(np.int32),
        "uniq": sk[heads].astype(np.int32),
        "counts": np.diff(seg_start).astype(np.int32),
        "seg_start": seg_start.astype(np.int32),
        "num_segments": len(heads),
        "err": bool(np.any(key == vocab)),
    }


def route_bruteforce(ids, vocab: int) -> dict:
    """The same result with plain Python (small inputs): ``sorted`` is stable by
    language guarantee; blocks are found by walking the sorted keys."""
    key = [int(k) for k in _keys(ids, vocab)]
    n = len(key)
    perm = sorted(range(n), key=lambda i: key[i])
    sk = [key[i] for i in perm]
    inv = [0] * n
    for s, i in enumerate(perm):
        inv[i] = s
    uniq, counts, starts = [], [], []
    for s in range(n):
        if s == 0 or sk[s] != sk[s - 1]:
            uniq.append(sk[s])
            starts.append(s)
            counts.append(0)
        counts[-1] += 1
    starts.append(n)
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return {"perm": i32(perm), "sorted_ids": i32(sk), "inv_perm": i32(inv),
            "uniq": i32(uniq), "counts": i32(counts), "seg_start": i32(starts),
            "num_segments": len(uniq), "err": any(k == vocab for k in key)}
