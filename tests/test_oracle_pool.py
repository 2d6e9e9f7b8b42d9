"""The worker pool the GPU parity tests use to run the oracle over many rows
returns exactly what one in-process oracle call returns."""

import numpy as np

import oracle
from synth import make_kv_cache, make_query, make_workload
from tests.helpers import compact_oracle_inputs, oracle_positions, q_f64
from tests.oracle_pool import sparse_attention_rows


def test_pool_equals_one_oracle_call():
    wl = make_workload("C4s", kv_dtype="fp8")
    cache = make_kv_cache(wl, "cpu")
    q = q_f64(make_query(wl, "cpu"))
    req, pos = oracle_positions(wl)
    rows = np.arange(0, wl.total_q, 3)
    oc, bt, _, _ = compact_oracle_inputs(wl, cache, rows)
    want = oracle.sparse_attention(q, oc, wl.topk, bt, req, pos, wl.softmax_scale, rows=rows)
    got = sparse_attention_rows(oc, bt, q[rows], wl.topk[rows], req[rows], pos[rows], wl.softmax_scale,
                                workers=2, chunk=40, min_pool_rows=0)
    assert got.shape == want.shape
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
