"""The allocation-free decode entry point (msa_sparse_decode_noalloc, for
callers that cannot allocate) against msa_sparse_decode with a workspace:
two calls in a row through the C ABI, the second on a smaller input, each
bit-identical to the workspace call (same kernels, same split count), and
within the attention tolerance of the oracle."""

import numpy as np
import pytest
import torch

import oracle
import block_sparse_paged_query_amd as msa
from synth import make_kv_cache, make_query, make_workload
from tests.helpers import attention_within_tolerance, compact_oracle_inputs, oracle_positions, q_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV, torch.int32)


def _case(name, **kw):
    wl = make_workload(name, **kw)
    cache = make_kv_cache(wl, DEV)
    q = make_query(wl, DEV)
    ks = vs = None
    if wl.kv_dtype != "bf16":
        ks = torch.tensor([cache["k_scale"]], dtype=torch.float32, device=DEV)
        vs = torch.tensor([cache["v_scale"]], dtype=torch.float32, device=DEV)
    kv = msa.KVCache(wl.kv_dtype, cache["k_pages"], cache["v_pages"], wl.num_kv_heads, wl.head_dim,
                     wl.block_page_stride, ks, vs)
    return wl, cache, q, kv


def test_noalloc_decode_matches_workspace_decode():
    assert msa.load_library().msa_decode_noalloc_scratch_bytes() >= 9 << 20
    # the larger input first (many splits: 3 requests x 8 kv heads), then a
    # smaller one (2 requests x 1 kv head), so the second call reuses a scratch
    # array the first one filled
    for name, kw in (("C2s", dict(dql=2)), ("C1", {})):
        wl, cache, q, kv = _case(name, **kw)
        topk, bt, seq = _dev(wl.topk), _dev(wl.block_table), _dev(wl.seq_lens)
        want = msa.msa_sparse_decode(q, kv, topk, bt, seq, wl.softmax_scale, decode_query_len=wl.decode_query_len)
        got = torch.full_like(q, float("nan"))
        msa.msa_sparse_decode_noalloc(q, kv, topk, bt, seq, wl.softmax_scale, out=got,
                                      decode_query_len=wl.decode_query_len)
        torch.cuda.synchronize()
        assert torch.equal(got, want), name
        req, pos = oracle_positions(wl)
        rows = np.arange(wl.total_q)
        oc, obt, _, _ = compact_oracle_inputs(wl, cache, rows)
        ref = oracle.sparse_attention(q_f64(q), oc, wl.topk, obt, req, pos, wl.softmax_scale)
        ok, err, _, _ = attention_within_tolerance(got.float().cpu().numpy(), ref)
        assert ok, f"{name}: max abs error {err}"
