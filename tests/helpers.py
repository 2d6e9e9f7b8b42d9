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
    layout = cache.get("layout", "page16")
    k = np_bytes(cache["k_pages"])
    v = None if layout == "rows128" else np_bytes(cache["v_pages"])
    if wl.kv_dtype == "bf16":
        k = k.view(np.uint16)
        v = None if v is None else v.view(np.uint16)
    return oracle.PagedKVCache(wl.kv_dtype, k, v, wl.num_kv_heads, wl.head_dim,
                               wl.block_page_stride, cache["k_scale"], cache["v_scale"], layout=layout)


def oracle_positions(wl):
    if wl.mode == "decode":
        return oracle.decode_positions(wl.seq_lens, wl.decode_query_len)
    return oracle.prefill_positions(wl.cu_seqlens_q, wl.seq_lens, wl.total_q)


def q_f64(q):
    return q.detach().float().cpu().numpy().astype(np.float64)


def rows_blocks(wl, rows, pos, req):
    """Physical blocks the oracle's masks of `rows` touch."""
    need = set()
    for i in rows:
        toks = oracle.token_mask(wl.topk[i], int(pos[i]), wl.block_table.shape[1])
        for b in set((toks // 128).tolist()):
            need.add(int(wl.block_table[req[i], b]))
    return sorted(need)


def compact_oracle_inputs(wl, cache, rows):
    """Oracle cache holding only the blocks `rows` read, plus a remapped block table.

    The pages of each needed physical block (all block_page_stride of them, so
    V pages of a packed layout come along) are copied from the device in one
    gather; block ids are renumbered densely.  Attention is invariant to that
    renumbering (pinned in the oracle tests).
    """
    req, pos = oracle_positions(wl)
    need = rows_blocks(wl, rows, pos, req)
    stride = wl.block_page_stride
    remap = np.zeros(wl.num_phys_blocks, dtype=np.int64)
    remap[need] = np.arange(len(need))
    if cache.get("layout", "page16") == "rows128":
        page_idx = np.asarray(need, dtype=np.int64)          # one page per block
    else:
        page_idx = (np.asarray(need, dtype=np.int64)[:, None] * stride + np.arange(stride)[None, :]).reshape(-1)
    idx = torch.from_numpy(page_idx).to(cache["k_pages"].device)
    small = dict(cache)
    small["k_pages"] = cache["k_pages"].index_select(0, idx)
    if cache["v_pages"] is not None:
        small["v_pages"] = cache["v_pages"].index_select(0, idx)
    bt = remap[wl.block_table]
    return oracle_cache(wl, small), bt, req, pos


def attention_within_tolerance(got, want, atol=1e-2):
    """Check bf16 attention outputs against fp64 oracle values.

    |got - want| <= atol wherever |want| < 4.  From 4 up, neighbouring bf16
    values lie 1/32 or more apart, so the rounding of the output alone can
    exceed atol there; the bound is then atol plus half a bf16 spacing at
    |want| (the compute error allowed below 4, plus round-to-nearest of the
    result).  Returns (ok, max error where |want| < 4, number of elements
    with |want| >= 4, max error relative to their bound).
    """
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    big = np.abs(want) >= 4.0
    half_spacing = np.exp2(np.floor(np.log2(np.where(big, np.abs(want), 1.0))) - 8)
    bound = np.where(big, atol + half_spacing, atol)
    ok = bool((err <= bound).all())
    small_err = float(err[~big].max()) if (~big).any() else 0.0
    big_ratio = float((err[big] / bound[big]).max()) if big.any() else 0.0
    return ok, small_err, int(big.sum()), big_ratio
