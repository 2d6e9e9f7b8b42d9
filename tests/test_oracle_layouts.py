"""Pins of the oracle's cache layouts (CPU only).

The K|V-interleaved 128-token pages ([FI] =
vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer,
MiniMaxM3SparseFlashInferBackend.supported_kv_cache_layouts: one dense
(pages, kv heads, 128, 2 * head_dim) tensor, K and V interleaved per row):
the oracle's reading is checked against arrays built by hand from that
description, and the generator's re-layout of a 16-token-page cache against
the oracle reading both layouts.
"""

import numpy as np
import pytest

import oracle
from synth import make_workload, make_kv_cache, make_query, rows128_cache, written_blocks
from tests.helpers import oracle_cache, oracle_positions, q_f64


def test_rows128_reads_k_then_v_of_each_row():
    rng = np.random.default_rng(5)
    nb, Hkv, D = 3, 2, 16
    # random finite bf16 bit patterns (sign, exponent 0x70..0x8f, mantissa)
    def codes(shape):
        return ((rng.integers(0, 2, shape) << 15) | (rng.integers(0x70, 0x90, shape) << 7)
                | rng.integers(0, 128, shape)).astype(np.uint16)
    K = codes((nb, 128, Hkv, D))       # token t of block b, kv head h
    V = codes((nb, 128, Hkv, D))
    pages = np.empty((nb, Hkv, 128, 2 * D), dtype=np.uint16)
    for b in range(nb):
        for h in range(Hkv):
            for t in range(128):
                pages[b, h, t, :D] = K[b, t, h]
                pages[b, h, t, D:] = V[b, t, h]
    cache = oracle.PagedKVCache("bf16", pages, None, Hkv, D, 8, layout="rows128")
    bt_row = np.array([2, 0, 1])       # logical block i lives in page bt_row[i]
    tok = np.arange(3 * 128)
    k, v = oracle.gather_tokens(cache, bt_row, tok)
    phys = bt_row[tok // 128]
    assert np.array_equal(k, oracle.bf16_value(K[phys, tok % 128]))
    assert np.array_equal(v, oracle.bf16_value(V[phys, tok % 128]))


def test_rows128_rejects_nvfp4():
    with pytest.raises(ValueError):
        oracle.PagedKVCache("nvfp4", np.zeros((1, 2, 9 * 128), np.uint8), None, 1, 128, layout="rows128")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("layers", [1, 3])
def test_rows128_cache_holds_the_same_tokens(kv_dtype, layers):
    wl = make_workload("C2s", kv_dtype=kv_dtype, seed=71)
    cache = make_kv_cache(wl, "cpu")
    rows = rows128_cache(cache, wl, layers=layers, layer=layers // 2)
    assert rows["k_pages"].shape == (wl.num_phys_blocks, wl.num_kv_heads, 128, 2 * wl.head_dim *
                                     (2 if kv_dtype == "bf16" else 1))
    assert rows["page_stride_bytes"] == layers * rows["k_pages"][0].numel()
    a, b = oracle_cache(wl, cache), oracle_cache(wl, rows)
    for (r, blk, n) in written_blocks(wl):
        pages = int(wl.block_table[r, blk]) * 8 + np.arange(n) // 16
        slots = np.arange(n) % 16
        for side in ("k", "v"):
            assert np.array_equal(a.read_tokens(side, pages, slots), b.read_tokens(side, pages, slots))


def test_rows128_attention_equals_page16():
    wl = make_workload("C3s", seed=72)
    cache = make_kv_cache(wl, "cpu")
    q = q_f64(make_query(wl, "cpu"))
    req, pos = oracle_positions(wl)
    a = oracle.sparse_attention(q, oracle_cache(wl, cache), wl.topk, wl.block_table, req, pos, wl.softmax_scale)
    b = oracle.sparse_attention(q, oracle_cache(wl, rows128_cache(cache, wl)), wl.topk, wl.block_table, req, pos,
                                wl.softmax_scale)
    assert np.array_equal(a, b)
