"""The C-ABI library on the CPU: it loads, exports every symbol include/msa.h
declares, and rejects bad arguments before touching the GPU (no kernel runs:
each call below fails validation, which precedes any HIP call)."""

import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_paged_query_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(msa.library_path()), reason="libmsa.so not built")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MSA_API\s+[\w\s\*]+?\b(msa_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared()
    for n in ["msa_build_sparse_block_table", "msa_sparse_decode", "msa_sparse_prefill",
              "msa_insert_index_cache", "msa_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(msa.library_path())
    for n in declared():
        assert hasattr(lib, n), n


def _lib():
    return msa.load_library()


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _table(**kw):
    args = dict(topk=FAKE, topk_row_stride=4, topk_k=4, total_q=3, block_table=FAKE, bt_row_stride=8, bt_cols=8,
                num_reqs=2, seq_lens=FAKE, dql=1, req_id=None, abs_pos=None, bps=8, sbt=FAKE, sbt_stride=32,
                ctx=FAKE)
    args.update(kw)
    return _lib().msa_build_sparse_block_table(*args.values(), None)


def test_table_rejects_row_count_mismatch():
    # decode-mode tables need one top-k row per (request, query token)
    assert _table(total_q=3, num_reqs=2, dql=1) == 1     # MSA_ERR_INVALID_ARGUMENT
    assert b"top-k rows for" in _lib().msa_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(topk_k=0), 2), (dict(topk_k=5000), 2), (dict(topk_row_stride=2), 1), (dict(bt_row_stride=4), 1),
    (dict(sbt_stride=16), 1), (dict(req_id=FAKE), 1), (dict(dql=0, total_q=0), 1), (dict(bps=0), 1),
])
def test_table_argument_errors(kw, status):
    assert _table(**kw) == status


def test_empty_inputs_are_noops():
    assert _table(total_q=0, num_reqs=0) == 0
    assert _lib().msa_insert_index_cache(FAKE, 1, 1, 0, 128, 0, FAKE, 1, 1, 1, 4, 16, FAKE, 1, None) == 0


def test_index_cache_needs_contiguous_head_dim():
    st = _lib().msa_insert_index_cache(FAKE, 128, 1, 5, 128, 0, FAKE, 128 * 16, 128, 2, 4, 16, FAKE, 1, None)
    assert st == 1 and b"along the key dimension, 1 needed" in _lib().msa_last_error()


def _kv(**kw):
    d = dict(kv_dtype=msa.MSA_BF16, num_kv_heads=8, head_dim=128, block_page_stride=8, k_pages=0x1000,
             v_pages=0x2000, page_stride_bytes=8 * 16 * 128 * 2, num_pages=64, k_scale=None, v_scale=None,
             kv_layout=0)
    d.update(kw)
    return msa._KV(*d.values())


def _decode(kv, **kw):
    args = dict(q=FAKE, q_dtype=0, num_reqs=4, dql=1, hq=64, kv=ctypes.byref(kv), topk=FAKE, topk_stride=16,
                topk_k=16, bt=FAKE, bt_stride=64, bt_cols=64, seq=FAKE, scale=0.1, out=FAKE, ws=None, ws_bytes=0)
    args.update(kw)
    return _lib().msa_sparse_decode(*args.values(), None)


@pytest.mark.parametrize("kvkw,kw,status", [
    (dict(head_dim=96), {}, 2),
    (dict(kv_dtype=msa.MSA_NVFP4, head_dim=64, page_stride_bytes=2 * 8 * 9 * 64), {}, 2),
    (dict(kv_dtype=7), {}, 2),
    ({}, dict(hq=60), 1),
    ({}, dict(hq=8 * 32), 2),
    (dict(block_page_stride=12), {}, 1),
    (dict(page_stride_bytes=100), {}, 1),
    ({}, dict(q_dtype=msa.MSA_FP16), 2),
    ({}, dict(topk_k=2048), 2),
    ({}, dict(q=ctypes.c_void_p(0x1001)), 1),
    ({}, dict(scale=float("nan")), 1),
])
def test_decode_argument_errors(kvkw, kw, status):
    assert _decode(_kv(**kvkw), **kw) == status


def test_decode_empty_batch_is_noop():
    assert _decode(_kv(), num_reqs=0) == 0


ROWS128 = dict(kv_layout=1, v_pages=None, page_stride_bytes=8 * 128 * 2 * 128 * 2)


@pytest.mark.parametrize("kvkw,status", [
    (dict(ROWS128), 0),                                          # valid (empty batch: nothing runs)
    (dict(ROWS128, v_pages=0x1000 + 256), 0),                    # V view of the same buffer
    (dict(ROWS128, v_pages=0x2000), 1),                          # V elsewhere
    (dict(ROWS128, block_page_stride=16), 1),                    # one page per block
    (dict(ROWS128, page_stride_bytes=8 * 16 * 128 * 2), 1),     # smaller than a 128-token page
    (dict(ROWS128, page_stride_bytes=8 * 128 * 2 * 128 * 2 + 4096), 1),   # not a multiple of 16 rows
    (dict(ROWS128, page_stride_bytes=3 * 8 * 128 * 2 * 128 * 2), 0),      # three layers, block-outer
    (dict(ROWS128, kv_dtype=msa.MSA_NVFP4, page_stride_bytes=1 << 20), 2),
    (dict(kv_layout=2), 1),
])
def test_rows128_layout_checks(kvkw, status):
    assert _decode(_kv(**kvkw), num_reqs=0) == status
    if status:
        assert _decode(_kv(**kvkw)) == status


def test_prefill_rejects_unsupported_shapes():
    # validation runs before any HIP call, so fake device pointers are safe
    kv = _kv(kv_dtype=msa.MSA_FP8_E4M3FN, page_stride_bytes=8 * 16 * 128)
    fp16_q = _lib().msa_sparse_prefill(FAKE, 1, 10, 64, ctypes.byref(kv), FAKE, 16, 16, FAKE, 64, 64, 1, FAKE, FAKE,
                                       0.1, FAKE, None, 0, None)
    assert fp16_q == 2
    kv96 = _kv(head_dim=96, page_stride_bytes=8 * 16 * 96 * 2)
    d96 = _lib().msa_sparse_prefill(FAKE, 0, 10, 64, ctypes.byref(kv96), FAKE, 16, 16, FAKE, 64, 64, 1, FAKE, FAKE,
                                    0.1, FAKE, None, 0, None)
    assert d96 == 2


def _mixed(kv, **kw):
    args = dict(q=FAKE, q_dtype=0, num_tokens=10, hq=64, kv=ctypes.byref(kv), topk=FAKE, topk_stride=16, topk_k=16,
                nd=4, dql=2, dbt=FAKE, dbt_stride=64, dbt_cols=64, dsl=FAKE, npre=1, pbt=FAKE, pbt_stride=64,
                pbt_cols=64, pcu=FAKE, psl=FAKE, scale=0.1, out=FAKE, ws=None, ws_bytes=0)
    args.update(kw)
    return _lib().msa_sparse_attention(*args.values(), None)


def test_mixed_batch_validates_both_parts_first():
    # every check runs before any HIP call, so fake device pointers are safe
    kv = _kv()
    assert _mixed(kv, nd=11) == 1                 # more decode rows than rows
    assert _mixed(kv, nd=3) == 1                  # not a multiple of decode_query_len
    assert _mixed(kv, dsl=None) == 1              # decode part without seq_lens
    assert _mixed(kv, pcu=None) == 1              # prefill part without cu_seqlens_q
    assert _mixed(kv, q_dtype=1) == 2             # fp16 queries are not served
    assert _mixed(kv, num_tokens=0, nd=0) == 0    # empty batch: nothing to do


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(msa, "_lib", None)
    monkeypatch.setattr(msa, "library_path", lambda: str(tmp_path / "libmsa.so"))
    with pytest.raises(RuntimeError, match="not built"):
        msa.load_library()


def test_binding_rejects_host_tensors():
    # host pointers must never reach the kernels
    import torch
    from synth import make_workload, make_kv_cache, make_query
    wl = make_workload("C1")
    cache = make_kv_cache(wl, "cpu")
    q = make_query(wl, "cpu")
    kv = msa.KVCache(wl.kv_dtype, cache["k_pages"], cache["v_pages"], wl.num_kv_heads, wl.head_dim)
    t = lambda x: torch.from_numpy(x)
    with pytest.raises(ValueError, match="GPU"):
        msa.msa_sparse_decode(q, kv, t(wl.topk), t(wl.block_table), t(wl.seq_lens), wl.softmax_scale)
    with pytest.raises(ValueError, match="GPU"):
        kv._struct()
    with pytest.raises(ValueError, match="GPU"):
        msa.msa_build_sparse_block_table(t(wl.topk), t(wl.block_table), seq_lens=t(wl.seq_lens))
    with pytest.raises(ValueError, match="GPU"):
        msa.msa_query_token_positions(t(np.array([0, 3], np.int32)), t(np.array([0], np.int32)), 3)


def test_binding_rejects_host_or_strided_workspaces():
    # the library writes up to workspace_bytes bytes from the workspace
    # pointer on the GPU: a host tensor or a strided view must not reach it
    import torch
    from synth import make_workload, make_kv_cache, make_query
    wl = make_workload("C4s")
    cache = make_kv_cache(wl, "cpu")
    kv = msa.KVCache(wl.kv_dtype, cache["k_pages"], cache["v_pages"], wl.num_kv_heads, wl.head_dim)
    q = make_query(wl, "cpu")
    t = lambda x: torch.from_numpy(x)
    args = (q, kv, t(wl.topk), t(wl.block_table), t(wl.cu_seqlens_q), t(wl.seq_lens), wl.softmax_scale)
    with pytest.raises(ValueError, match="GPU"):
        msa.msa_sparse_prefill(*args, workspace=torch.empty(64, dtype=torch.uint8))
    with pytest.raises(TypeError, match="torch.Tensor"):
        msa.msa_sparse_prefill(*args, workspace=bytearray(64))
    with pytest.raises(ValueError, match="GPU"):
        msa.msa_sparse_decode(q, kv, t(wl.topk), t(wl.block_table), t(wl.seq_lens), wl.softmax_scale,
                              workspace=torch.empty(64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        msa.msa_sparse_attention(q, kv, t(wl.topk), 0, wl.softmax_scale, workspace=torch.empty(64, dtype=torch.uint8))


def test_binding_rejects_pages_that_are_not_dense():
    import torch
    kp = torch.zeros((4, 2, 16, 256), dtype=torch.bfloat16)[..., :128]    # a head_dim slice of wider rows
    kv = msa.KVCache("bf16", kp, kp, 2, 128)
    with pytest.raises(ValueError, match="dense"):
        kv._struct()


def test_binding_rejects_short_block_tables():
    # the kernels read block_table row r for every request r (and the decode
    # table builder seq_lens[r] for every block_table row): shapes that would
    # send them past a buffer's end are refused before any device check
    import torch
    from synth import make_workload
    wl = make_workload("C2s")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    topk, bt, seq = t(wl.topk), t(wl.block_table), t(wl.seq_lens)
    q = torch.zeros((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16)
    kv = msa.KVCache("bf16", torch.zeros((8, 8, 16, 128), dtype=torch.bfloat16), None, 8, 128)
    with pytest.raises(ValueError, match="rows for 3 requests"):
        msa.msa_sparse_decode(q, kv, topk, bt[:2], seq, wl.softmax_scale)
    with pytest.raises(ValueError, match="requests, block_table"):
        msa.msa_build_sparse_block_table(topk, bt, seq_lens=seq[:2])
    with pytest.raises(ValueError, match="need seq_lens"):
        msa.msa_build_sparse_block_table(topk, bt)
    pre = make_workload("C4s")
    cu, pseq = t(pre.cu_seqlens_q), t(pre.seq_lens)
    qp = torch.zeros((pre.total_q, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="rows for 2 requests"):
        msa.msa_sparse_prefill(qp, kv, t(pre.topk), t(pre.block_table)[:1], cu, pseq, pre.softmax_scale)
    both = torch.cat([q, qp])
    with pytest.raises(ValueError, match="decode_block_table has 2 rows"):
        msa.msa_sparse_attention(both, kv, t(np.concatenate([wl.topk, pre.topk])), wl.total_q, 0.1,
                                 decode_block_table=bt[:2], decode_seq_lens=seq,
                                 prefill_block_table=t(pre.block_table), prefill_cu_seqlens_q=cu,
                                 prefill_seq_lens=pseq)
    with pytest.raises(ValueError, match="prefill_block_table has 1 rows"):
        msa.msa_sparse_attention(both, kv, t(np.concatenate([wl.topk, pre.topk])), wl.total_q, 0.1,
                                 decode_block_table=bt, decode_seq_lens=seq,
                                 prefill_block_table=t(pre.block_table)[:1], prefill_cu_seqlens_q=cu,
                                 prefill_seq_lens=pseq)


def test_index_cache_binding_checks():
    import torch
    k = torch.zeros((4, 8), dtype=torch.bfloat16)
    c = torch.zeros((2, 4, 8), dtype=torch.bfloat16)
    s = torch.zeros(4, dtype=torch.int64)
    msa.msa_insert_index_cache(k[:0], c, s[:0])                   # empty input: nothing to do
    with pytest.raises(ValueError, match="3-D"):
        msa.msa_insert_index_cache(k, c[0], s)
    with pytest.raises(ValueError, match="elements"):
        msa.msa_insert_index_cache(torch.zeros((4, 6), dtype=torch.bfloat16), c, s)
    with pytest.raises(ValueError, match="slots for"):
        msa.msa_insert_index_cache(k, c, s[:3])
    with pytest.raises(TypeError, match="int64"):
        msa.msa_insert_index_cache(k, c, s.int())
    with pytest.raises(ValueError, match="contiguous last"):
        msa.msa_insert_index_cache(k, torch.zeros((2, 8, 4), dtype=torch.bfloat16).transpose(1, 2), s)
    with pytest.raises(ValueError, match="GPU"):
        msa.msa_insert_index_cache(k, c, s)                           # host tensors never reach a kernel


def test_prefill_workspace_covers_every_query_tile():
    # msa_sparse_prefill keeps one 32-byte row order per 32-row query tile
    # (a request of n rows has ceil(n / 32) tiles).  The size it asks for
    # must cover any split of total_q rows into requests, down to one row each.
    assert msa.msa_prefill_workspace_size(0, 64, 128, 16) == 0
    rng = np.random.default_rng(5)
    for total in (1, 31, 32, 33, 1000, 22592):
        splits = [[total], [1] * total, rng.multinomial(total, np.ones(7) / 7).tolist(),
                  [31] * (total // 31) + [total % 31]]
        for lens in splits:
            tiles = sum((n + 31) // 32 for n in lens)
            assert 32 * tiles <= msa.msa_prefill_workspace_size(total, 64, 128, 16), (total, lens[:5])
