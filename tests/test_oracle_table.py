"""Pins of the oracle's page-16 table and context length (CPU only).

The table follows [SPA] = vllm.models.minimax_m3.amd.ops.sparse_pa,
``_write_sparse_block_table_row_from_values``.  The pages print no worked
example, so the examples below are derived by hand from that routine, each
step written out; the closed forms and the mask cross-check pin the rest.
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from synth import make_workload
from tests.helpers import oracle_positions

BT_ROW = [9, 3, 12, 0, 7, 1, 13, 4]  # logical block -> physical block, 8 blocks


def _pages(phys, stride=8):
    return list(range(phys * stride, phys * stride + 8))


# Hand-derived rows.  Position 999 (a sequence of 1000, one decode token):
# own block 999 // 128 = 7, causal length 1000, tail tokens 1000 - 7*128 = 104.
@pytest.mark.parametrize("topk,abs_pos,stride,expect_row,expect_ctx", [
    # full 5 -> slot 0 (bt 1), full 2 -> slot 1 (bt 12), tail 7 -> slot 2 (bt 4);
    # ctx = 2 full * 128 + 104 tail tokens
    ([5, 7, -1, 2], 999, 8, _pages(1) + _pages(12) + _pages(4) + [0] * 8, 360),
    # same row at block stride 16: page ids are bt * 16 + j
    ([5, 7, -1, 2], 999, 16, _pages(1, 16) + _pages(12, 16) + _pages(4, 16) + [0] * 8, 360),
    # own block absent: two full blocks, ctx = min(2 * 128, 1000)
    ([5, 2, -1, -1], 999, 8, _pages(1) + _pages(12) + [0] * 16, 256),
    # 8 is in the future and dropped; full 3 (bt 0), full 1 (bt 3), tail 7 (bt 4)
    ([8, 7, 3, 1], 999, 8, _pages(0) + _pages(3) + _pages(4) + [0] * 8, 360),
    # padded row: negative position, nothing is valid
    ([5, 7, -1, 2], -1, 8, [0] * 32, 0),
    # last token of block 0: own block 0 is a full-length tail of 128 tokens
    ([0, -1, -1, -1], 127, 8, _pages(9) + [0] * 24, 128),
    # first token of block 1: full 0 (bt 9), tail 1 (bt 3) holding one token
    ([1, 0, -1, -1], 128, 8, _pages(9) + _pages(3) + [0] * 16, 129),
    # position 0: every earlier id is in the future; only the 1-token tail
    ([3, 0, 2, 1], 0, 8, _pages(9) + [0] * 24, 1),
])
def test_hand_derived_rows(topk, abs_pos, stride, expect_row, expect_ctx):
    row, ctx = oracle.sparse_table_row(np.array(topk), np.array(BT_ROW), abs_pos, stride)
    assert row.tolist() == expect_row
    assert ctx == expect_ctx


def test_repeated_ids_are_refused():
    with pytest.raises(ValueError):
        oracle.sparse_table_row(np.array([2, 2, -1, -1]), np.array(BT_ROW), 999)


def _table(wl, stride=8, bt=None):
    req, pos = oracle_positions(wl)
    return oracle.sparse_block_table(wl.topk, wl.block_table if bt is None else bt, req, pos, stride)


def test_tiny_decode_context_lengths():
    # 2 requests of 1000 and 700 tokens, k = 4 (own + 3 earlier):
    # ctx = 3 * 128 + (999 % 128) + 1 = 488 and 3 * 128 + (699 % 128) + 1 = 444
    wl = make_workload("C1")
    _, ctx = _table(wl)
    assert ctx.tolist() == [488, 444]


@pytest.mark.parametrize("name", ["C2", "C3", "C5"])
def test_decode_closed_form(name):
    # every decode row of these workloads selects its own block and k-1 earlier
    # ones (sequences are long), so ctx = (k-1) * 128 + pos % 128 + 1
    wl = make_workload(name)
    req, pos = oracle_positions(wl)
    _, ctx = _table(wl)
    k = wl.topk_k
    assert (ctx == (k - 1) * 128 + pos % 128 + 1).all()


def test_prefill_total_context():
    # 4 requests of 2048 / 4096 / 8192 / 8192 new tokens, k = 16, no context:
    # a token at position p sees min(15, p // 128) full blocks plus p % 128 + 1
    # tail tokens.  Summed in closed form per 128-token block b of a request:
    # 128 * min(15, b) * 128 + (1 + ... + 128).
    def per_request(q):
        return sum(128 * min(15, b) * 128 + 128 * 129 // 2 for b in range(q // 128))
    closed = sum(per_request(q) for q in (2048, 4096, 8192, 8192))
    assert closed == 36_842_496
    wl = make_workload("C4")
    _, ctx = _table(wl)
    assert int(ctx.sum()) == closed
    assert (ctx[-64:] == 0).all()          # the 64 padded rows


def _mask_matches_table(wl, stride=8):
    req, pos = oracle_positions(wl)
    sbt, ctx = _table(wl, stride)
    for i in range(wl.total_q):
        toks = oracle.token_mask(wl.topk[i], int(pos[i]), wl.block_table.shape[1])
        assert ctx[i] == len(toks)
        # the first ctx slots address exactly the mask's tokens, through the block table
        bt = wl.block_table[req[i]]
        want = {(int(bt[j // 128]) * stride + (j % 128) // 16, j % 16) for j in toks}
        got = {(int(sbt[i, s // 16]), s % 16) for s in range(int(ctx[i]))}
        assert got == want
        assert (sbt[i, 8 * ((int(ctx[i]) + 127) // 128):] == 0).all()


@pytest.mark.parametrize("name", ["C1", "C2s", "C3s", "C4s", "C5s"])
def test_table_addresses_the_mask(name):
    _mask_matches_table(make_workload(name))


def test_table_addresses_the_mask_stride16():
    _mask_matches_table(make_workload("C4s", block_page_stride=16), stride=16)


@pytest.mark.parametrize("name", ["C1", "C3s", "C4s"])
def test_stride16_equals_rebased_table(name):
    # [SPA] minimax_m3_rebase_block_table_to_page16 scales the table by the
    # two sides a block holds; that table at stride 8 equals the stride-16 table.
    wl = make_workload(name)
    a, ca = _table(wl, stride=16)
    b, cb = _table(wl, stride=8, bt=wl.block_table * 2)
    assert (a == b).all() and (ca == cb).all()


@settings(max_examples=200, deadline=None)
@given(st.data())
def test_random_rows_mask_and_order(data):
    nblk = data.draw(st.integers(1, 12))
    k = data.draw(st.integers(1, 10))
    abs_pos = data.draw(st.integers(-3, nblk * 128 - 1))
    ids = data.draw(st.lists(st.integers(0, nblk + 2), min_size=0, max_size=k, unique=True))
    row = np.array(ids + [-1] * (k - len(ids)))
    row = np.array(data.draw(st.permutations(row.tolist())))
    bt = np.array(data.draw(st.permutations(list(range(nblk)))))
    sbt, ctx = oracle.sparse_table_row(row, bt, abs_pos)
    toks = oracle.token_mask(row, abs_pos, nblk)
    assert ctx == len(toks)
    # order of the row changes the slot order of full blocks only
    sbt2, ctx2 = oracle.sparse_table_row(row[::-1].copy(), bt, abs_pos)
    assert ctx2 == ctx
    assert sorted(sbt2.tolist()) == sorted(sbt.tolist())
    # the tail block, when present, sits in the last used slot
    if abs_pos >= 0 and (abs_pos // 128) in set(row.tolist()) and abs_pos // 128 < nblk:
        n_used = (ctx + 127) // 128
        assert sbt[(n_used - 1) * 8] == bt[abs_pos // 128] * 8


def test_prefill_positions_with_context():
    # request 0: 300 new tokens, no context; request 1: 517 new tokens after 200
    wl = make_workload("C4s")
    req, pos = oracle.prefill_positions(wl.cu_seqlens_q, wl.seq_lens, wl.total_q)
    assert pos[0] == 0 and pos[299] == 299
    assert req[300] == 1 and pos[300] == 200 and pos[816] == 716
    assert (pos[817:] == -1).all() and len(pos) == 822


def test_decode_positions_right_aligned():
    req, pos = oracle.decode_positions(np.array([10, 7]), 4)
    assert req.tolist() == [0, 0, 0, 0, 1, 1, 1, 1]
    assert pos.tolist() == [6, 7, 8, 9, 3, 4, 5, 6]
