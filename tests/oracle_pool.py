"""Run the CPU oracle over many query rows in spawned worker processes.

Test plumbing only: the arithmetic is the oracle's own ``sparse_attention``,
called unchanged on contiguous row chunks (each row's output depends on that
row alone, so a chunk's result equals the same rows of one whole call).
Workers are spawned (a fresh interpreter, numpy only: no GPU context is
inherited or touched) and read the compacted cache from .npy files mapped
read-only.  BLAS runs one thread per worker.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import tempfile

import numpy as np

import oracle


def _worker(arg):
    (cache_dir, meta, q, topk, req, pos, scale) = arg
    from threadpoolctl import threadpool_limits

    kv_dtype, hkv, d, stride, ks, vs, layout = meta
    kp = np.load(os.path.join(cache_dir, "k.npy"), mmap_mode="r")
    vpath = os.path.join(cache_dir, "v.npy")
    vp = np.load(vpath, mmap_mode="r") if os.path.exists(vpath) else None
    bt = np.load(os.path.join(cache_dir, "bt.npy"))
    cache = oracle.PagedKVCache(kv_dtype, kp, vp, hkv, d, stride, ks, vs, layout=layout)
    with threadpool_limits(1):
        return oracle.sparse_attention(q, cache, topk, bt, req, pos, scale)


def default_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def sparse_attention_rows(oc, block_table, q_rows, topk_rows, req_rows, pos_rows, softmax_scale, workers=None,
                          chunk=64, min_pool_rows=2048):
    """The oracle's outputs [n, Hq, D] for n rows given row by row: q_rows [n,
    Hq, D] fp64, topk_rows [n, k], req_rows / pos_rows [n].  ``oc`` is an
    oracle.PagedKVCache, ``block_table`` the table its block ids follow.
    Up to ``min_pool_rows`` rows run in this process (a worker pool's start-up
    costs more than they do)."""
    n = len(req_rows)
    workers = default_workers() if workers is None else workers
    if n == 0:
        return np.zeros((0,) + q_rows.shape[1:])
    if workers <= 1 or n <= min_pool_rows:
        return oracle.sparse_attention(q_rows, oc, topk_rows, block_table, req_rows, pos_rows, softmax_scale)
    meta = (oc.kv_dtype, oc.num_kv_heads, oc.head_dim, oc.block_page_stride, oc.k_scale, oc.v_scale, oc.layout)
    with tempfile.TemporaryDirectory(prefix="oracle_pool_") as tmp:
        np.save(os.path.join(tmp, "k.npy"), np.ascontiguousarray(oc.k_pages))
        if oc.v_pages is not None:
            np.save(os.path.join(tmp, "v.npy"), np.ascontiguousarray(oc.v_pages))
        np.save(os.path.join(tmp, "bt.npy"), np.ascontiguousarray(block_table))
        args = [(tmp, meta, q_rows[s:s + chunk], topk_rows[s:s + chunk], req_rows[s:s + chunk],
                 pos_rows[s:s + chunk], softmax_scale) for s in range(0, n, chunk)]
        with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
            parts = list(ex.map(_worker, args))
    return np.concatenate(parts)
