"""Test plumbing shared by the CPU and GPU tests (no method arithmetic)."""

import numpy as np
import torch

import oracle


def np_bytes(t):
    return t.detach().cpu().contiguous().numpy()


def oracle_cache(wl, cache):
    """Wrap a synth cache (torch byte tensors, any device) for the oracle."""
    if wl.kv_dtype == "nvfp4":
        k = np_bytes(cache["k_pages"])
        return oracle.PagedKVCache("nvfp4", k, None, wl.num_kv_heads, wl.head_dim,
                                   wl.block_page_stride, cache["k_scale"], cache["v_scale"])
    k = np_bytes(cache["k_pages"])
    v = np_bytes(cache["v_pages"])
    if wl.kv_dtype == "bf16":
        k = k.view(np.uint16)
        v = v.view(np.uint16)
    return oracle.PagedKVCache(wl.kv_dtype, k, v, wl.num_kv_heads, wl.head_dim,
                               wl.block_page_stride, cache["k_scale"], cache["v_scale"])


def oracle_positions(wl):
    if wl.mode == "decode":
        return oracle.decode_positions(wl.seq_lens, wl.decode_query_len)
    return oracle.prefill_positions(wl.cu_seqlens_q, wl.seq_lens, wl.total_q)


def q_f64(q):
    return q.detach().float().cpu().numpy().astype(np.float64)
