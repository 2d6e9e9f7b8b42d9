"""Pins of the oracle's attention (CPU only).

* top-k naming every block reduces to dense causal attention, and top-k = the
  own block to block-local causal attention: both checked against torch's
  scaled_dot_product_attention in fp64 (a library routine, GQA through its
  enable_gqa convention);
* brute force: pure-Python loops with math.fsum on tiny shapes;
* invariants: order of a top-k row, permutation of the physical blocks, padded
  rows, the fp8 scale-folding identity of [FI] =
  vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer,
  MiniMaxM3SparseFlashInferImpl.forward.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import oracle
from synth import make_workload, make_kv_cache, make_query
from tests.helpers import oracle_cache, oracle_positions, q_f64


def _setup(name, **kw):
    wl = make_workload(name, **kw)
    cache = make_kv_cache(wl, "cpu")
    q = q_f64(make_query(wl, "cpu"))
    return wl, oracle_cache(wl, cache), q


def _all_blocks_topk(wl):
    mb = wl.block_table.shape[1]
    k = max(mb, 1)
    return np.tile(np.arange(k, dtype=np.int32), (wl.total_q, 1))


def _sdpa(q, K, V, mask, scale):
    # q [rows, Hq, D], K/V [n, Hkv, D], mask [rows, n] bool
    # tokens outside the mask may be unwritten (NaN); the library multiplies
    # masked weights by them, so give it zeros there
    K = np.where(mask.any(axis=0)[:, None, None], K, 0.0)
    V = np.where(mask.any(axis=0)[:, None, None], V, 0.0)
    qq = torch.from_numpy(q).permute(1, 0, 2)[None]
    kk = torch.from_numpy(K).permute(1, 0, 2)[None]
    vv = torch.from_numpy(V).permute(1, 0, 2)[None]
    out = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=torch.from_numpy(mask), scale=scale, enable_gqa=True)
    return out[0].permute(1, 0, 2).numpy()


def _request_rows(wl, req, r):
    return np.flatnonzero((req == r))


@pytest.mark.parametrize("name", ["C3s", "C4s"])
def test_all_blocks_is_dense_causal(name):
    wl = make_workload(name)
    wl.topk = _all_blocks_topk(wl)        # select every block of the table
    cache = oracle_cache(wl, make_kv_cache(wl, "cpu"))
    q = q_f64(make_query(wl, "cpu"))
    req, pos = oracle_positions(wl)
    got = oracle.sparse_attention(q, cache, wl.topk, wl.block_table, req, pos, wl.softmax_scale)
    for r in range(wl.num_reqs):
        rows = _request_rows(wl, req, r)
        rows = rows[pos[rows] >= 0]
        L = int(wl.seq_lens[r])
        K, V = oracle.gather_tokens(cache, wl.block_table[r], np.arange(L))
        mask = np.arange(L)[None, :] <= pos[rows][:, None]          # right-aligned causal
        want = _sdpa(q[rows], K, V, mask, wl.softmax_scale)
        np.testing.assert_allclose(got[rows], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["C2s", "C4s"])
def test_own_block_only_is_block_local_causal(name):
    wl = make_workload(name)
    req, pos = oracle_positions(wl)
    own = np.full((wl.total_q, wl.topk_k), -1, dtype=np.int32)
    own[:, 0] = np.where(pos >= 0, pos // 128, -1)
    wl.topk = np.where(pos[:, None] >= 0, own, -1).astype(np.int32)
    cache = oracle_cache(wl, make_kv_cache(wl, "cpu"))
    q = q_f64(make_query(wl, "cpu"))
    got = oracle.sparse_attention(q, cache, wl.topk, wl.block_table, req, pos, wl.softmax_scale)
    for r in range(wl.num_reqs):
        rows = _request_rows(wl, req, r)
        rows = rows[pos[rows] >= 0]
        L = int(wl.seq_lens[r])
        K, V = oracle.gather_tokens(cache, wl.block_table[r], np.arange(L))
        j = np.arange(L)[None, :]
        p = pos[rows][:, None]
        mask = (j <= p) & (j // 128 == p // 128)                     # block-diagonal causal
        want = _sdpa(q[rows], K, V, mask, wl.softmax_scale)
        np.testing.assert_allclose(got[rows], want, rtol=0, atol=1e-12)
    assert (got[pos < 0] == 0).all()


def _brute(q_row, toks, K, V, scale, Hkv):
    """Pure-Python softmax attention with exactly rounded sums."""
    Hq, D = len(q_row), len(q_row[0])
    G = Hq // Hkv
    out = []
    for h in range(Hq):
        g = h // G
        s = [scale * math.fsum(q_row[h][d] * K[t][g][d] for d in range(D)) for t in range(len(toks))]
        if not s:
            out.append([0.0] * D)
            continue
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        out.append([math.fsum(w[t] * V[t][g][d] for t in range(len(toks))) / z for d in range(D)])
    return out


def test_brute_force_tiny_decode():
    wl, cache, q = _setup("C1")
    req, pos = oracle_positions(wl)
    got = oracle.sparse_attention(q, cache, wl.topk, wl.block_table, req, pos, wl.softmax_scale)
    for i in range(wl.total_q):
        # the mask, rebuilt here by brute force over all tokens
        sel = set(int(b) for b in wl.topk[i] if b >= 0)
        toks = [j for j in range(int(pos[i]) + 1) if j // 128 in sel]
        K, V = oracle.gather_tokens(cache, wl.block_table[req[i]], np.array(toks))
        want = _brute(q[i].tolist(), toks, K.tolist(), V.tolist(), wl.softmax_scale, wl.num_kv_heads)
        np.testing.assert_allclose(got[i], np.array(want), rtol=0, atol=1e-12)


@settings(max_examples=25, deadline=None)
@given(st.data())
def test_brute_force_random_shapes(data):
    rng = np.random.default_rng(data.draw(st.integers(0, 2 ** 31)))
    Hkv = data.draw(st.sampled_from([1, 2]))
    G = data.draw(st.sampled_from([1, 2, 4]))
    D = data.draw(st.sampled_from([4, 8]))
    n = data.draw(st.integers(0, 40))
    scale = data.draw(st.floats(0.05, 2.0))
    q_row = rng.standard_normal((Hkv * G, D))
    K = rng.standard_normal((n, Hkv, D))
    V = rng.standard_normal((n, Hkv, D))
    got = oracle.attend_row(q_row, K, V, scale)
    want = _brute(q_row.tolist(), list(range(n)), K.tolist(), V.tolist(), scale, Hkv)
    np.testing.assert_allclose(got, np.array(want).reshape(got.shape), rtol=0, atol=1e-12)


def test_topk_order_invariance():
    wl, cache, q = _setup("C3s")
    req, pos = oracle_positions(wl)
    a = oracle.sparse_attention(q, cache, wl.topk, wl.block_table, req, pos, wl.softmax_scale)
    rng = np.random.default_rng(7)
    shuffled = np.array([rng.permutation(r) for r in wl.topk])
    b = oracle.sparse_attention(q, cache, shuffled, wl.block_table, req, pos, wl.softmax_scale)
    assert (a == b).all()


def test_physical_block_permutation_invariance():
    wl, cache, q = _setup("C2s")
    req, pos = oracle_positions(wl)
    a = oracle.sparse_attention(q, cache, wl.topk, wl.block_table, req, pos, wl.softmax_scale)
    # move physical block p to perm[p]: pages and block table together
    nb = wl.num_phys_blocks
    perm = np.random.default_rng(3).permutation(nb)
    page_of = (perm[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)     # old page -> new page
    kp = np.empty_like(cache.k_pages)
    vp = np.empty_like(cache.v_pages)
    kp[page_of] = cache.k_pages
    vp[page_of] = cache.v_pages
    moved = oracle.PagedKVCache(cache.kv_dtype, kp, vp, cache.num_kv_heads, cache.head_dim,
                                8, cache.k_scale, cache.v_scale)
    bt = perm[wl.block_table]
    b = oracle.sparse_attention(q, moved, wl.topk, bt, req, pos, wl.softmax_scale)
    assert (a == b).all()


def test_padded_rows_are_zero():
    wl, cache, q = _setup("C4s")
    req, pos = oracle_positions(wl)
    rows = np.flatnonzero(pos < 0)
    assert len(rows) == 5
    out = oracle.sparse_attention(q, cache, wl.topk, wl.block_table, req, pos, wl.softmax_scale, rows=rows)
    assert (out == 0).all()


def test_fp8_scale_folding_identity():
    # [FI] forward: a K descale multiplies each logit and a V descale each
    # output, so the two scales move out of the attention:
    # attn(q, s_k K, s_v V, tau) == s_v * attn(q, K, V, tau * s_k)
    rng = np.random.default_rng(11)
    q_row = rng.standard_normal((8, 16))
    K = rng.standard_normal((50, 2, 16))
    V = rng.standard_normal((50, 2, 16))
    s_k, s_v, tau = 0.0123, 0.0456, 0.25
    lhs = oracle.attend_row(q_row, s_k * K, s_v * V, tau)
    rhs = s_v * oracle.attend_row(q_row, K, V, tau * s_k)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=0)
