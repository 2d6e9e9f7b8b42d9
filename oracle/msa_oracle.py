"""fp64 CPU oracle: causal top-k block-sparse attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and plain on
purpose: sequential loops where the pages describe a data layout, the plain
mathematical definition where the method reaches one.

Page titles are abbreviated in citations:

* [FI]  vllm.models.minimax_m3.nvidia.sparse_attention_flashinfer
* [NV4] vllm.models.minimax_m3.amd.sparse_attention_nvfp4
* [SPA] vllm.models.minimax_m3.amd.ops.sparse_pa

Readings where the pages are silent are tagged "reading:".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "SPARSE_BLOCK_SIZE", "PAGE_SIZE", "PAGES_PER_SPARSE_BLOCK",
    "decode_positions", "prefill_positions",
    "sparse_table_row", "sparse_block_table",
    "token_mask",
    "bf16_value", "fp8_e4m3fn_value", "e2m1_value", "nvfp4_token_values",
    "PagedKVCache", "gather_tokens",
    "attend_row", "sparse_attention",
    "insert_index_cache",
]

# [FI] supported_kv_cache_layouts: a sparse block is a 128-token page of the
# SM90 layout; [SPA] _write_sparse_block_table_row_from_values divides
# positions by SPARSE_BLOCK_SIZE_C.  The value itself is not printed next to
# the name; reading: 128, the block size every page names.
SPARSE_BLOCK_SIZE = 128
# [SPA] minimax_m3_rebase_block_table_to_page16: the attend numbers pages of
# 16 tokens ("page-16").
PAGE_SIZE = 16
# [SPA] PAGES_PER_SPARSE_BLOCK is used but not printed; reading: 128 / 16.
PAGES_PER_SPARSE_BLOCK = SPARSE_BLOCK_SIZE // PAGE_SIZE


# ---------------------------------------------------------------------------
# O1. Row positions
# ---------------------------------------------------------------------------

def decode_positions(seq_lens, decode_query_len):
    """Request id and absolute position of every decode row.

    [FI] MiniMaxM3SparseFlashInferImpl.forward: the kernels keep the default
    q_offset, which right-aligns the decode tokens of a request with its
    sequence; [SPA] minimax_m3_build_sparse_block_table_decode: there are
    batch * decode_query_len rows, request-major.  So row j of request r sits
    at seq_lens[r] - decode_query_len + j (reading of "right-aligns").
    """
    req, pos = [], []
    for r, L in enumerate(seq_lens):
        for j in range(decode_query_len):
            req.append(r)
            pos.append(int(L) - decode_query_len + j)
    return np.asarray(req, dtype=np.int64), np.asarray(pos, dtype=np.int64)


def prefill_positions(cu_seqlens_q, seq_lens, total_q):
    """Request id and absolute position of every prefill row.

    [NV4] MiniMaxM3SparseRocmNvfp4MetadataBuilder.build derives a request id
    and absolute position per prefill token from cu_seqlens_q and the
    requests' context lengths; the body of that helper is not printed.
    Reading: the context length of request r is seq_lens[r] minus its new
    tokens, token t of the request sits at context + (t - cu_seqlens_q[r]),
    and rows past cu_seqlens_q[-1] are padding with position -1 and request 0
    ([SPA] _write_sparse_block_table_row_from_values: padded rows carry a
    negative position).
    """
    num_reqs = len(seq_lens)
    req = np.zeros(total_q, dtype=np.int64)
    pos = np.full(total_q, -1, dtype=np.int64)
    for r in range(num_reqs):
        start, end = int(cu_seqlens_q[r]), int(cu_seqlens_q[r + 1])
        context = int(seq_lens[r]) - (end - start)
        for t in range(start, end):
            req[t] = r
            pos[t] = context + (t - start)
    return req, pos


# ---------------------------------------------------------------------------
# O5. The page-16 sparse block table, written as sequential loops
# ---------------------------------------------------------------------------

def sparse_table_row(topk_row, bt_row, abs_pos, block_page_stride=PAGES_PER_SPARSE_BLOCK):
    """One query row's page-16 table row and attended context length.

    [SPA] _write_sparse_block_table_row_from_values.  The causal range of a
    row is its position plus one (empty when the position is negative); its
    own block is position // 128.  A selected id is kept when it is not a
    pad, not in the future and (reading) inside the request's block table.
    Kept ids before the own block are "full" blocks and go first, in the order
    they appear; the own block, if selected, is the "tail" and goes last.
    Every kept block expands to its 8 page ids
    block_table[blk] * block_page_stride + j; the rest of the row is zero.
    The context length is 128 per full block plus the tail's causal tokens
    when the own block was selected, else min(kept * 128, causal range).

    Precondition (reading): the non-negative ids of a row are distinct; the
    printed routine double-counts repeated ids, so the oracle refuses them.
    """
    k = len(topk_row)
    width = k * PAGES_PER_SPARSE_BLOCK
    row = [0] * width
    causal_len = max(int(abs_pos) + 1, 0)
    ids = [int(b) for b in topk_row if int(b) >= 0]
    if len(set(ids)) != len(ids):
        raise ValueError("top-k row repeats a block id; rows must hold distinct ids")
    if causal_len == 0:
        return np.asarray(row, dtype=np.int64), 0
    self_blk = int(abs_pos) // SPARSE_BLOCK_SIZE
    full, has_tail = [], False
    for blk in topk_row:
        blk = int(blk)
        if blk < 0 or blk > self_blk or blk >= len(bt_row):
            continue
        if blk < self_blk:
            full.append(blk)
        else:
            has_tail = True
    order = full + ([self_blk] if has_tail else [])
    n = 0
    for blk in order:
        for j in range(PAGES_PER_SPARSE_BLOCK):
            row[n] = int(bt_row[blk]) * block_page_stride + j
            n += 1
    if has_tail:
        tail_tokens = causal_len - self_blk * SPARSE_BLOCK_SIZE
        ctx = len(full) * SPARSE_BLOCK_SIZE + tail_tokens
    else:
        ctx = min(len(order) * SPARSE_BLOCK_SIZE, causal_len)
    return np.asarray(row, dtype=np.int64), ctx


def sparse_block_table(topk, block_table, req, abs_pos, block_page_stride=PAGES_PER_SPARSE_BLOCK):
    """All rows of the page-16 table: ([rows, 8k] page ids, [rows] ctx).

    [SPA] minimax_m3_build_sparse_block_table_decode / _prefill: one row per
    query token, looked up in its own request's block_table row.
    """
    rows = len(req)
    k = topk.shape[1]
    sbt = np.zeros((rows, k * PAGES_PER_SPARSE_BLOCK), dtype=np.int64)
    ctx = np.zeros(rows, dtype=np.int64)
    for i in range(rows):
        bt_row = block_table[int(req[i])] if abs_pos[i] >= 0 else block_table[0]
        sbt[i], ctx[i] = sparse_table_row(topk[i], bt_row, abs_pos[i], block_page_stride)
    return sbt, ctx


# ---------------------------------------------------------------------------
# O2. The explicit causal top-k token mask (the plain definition)
# ---------------------------------------------------------------------------

def token_mask(topk_row, abs_pos, max_blocks):
    """Logical token positions a row attends to, ascending.

    A row sees exactly the tokens j <= abs_pos whose 128-token block j // 128
    is one of its selected ids ([SPA] _write_sparse_block_table_row_from_values:
    ids past the own block are dropped and the own block is cut at the row's
    causal length; [FI] MiniMaxM3SparseFlashInferImpl.forward passes
    causal=True).  Negative positions see nothing.  Reading: ids outside the
    block table (>= max_blocks) are dropped.
    """
    if abs_pos < 0:
        return np.zeros(0, dtype=np.int64)
    blocks = {int(b) for b in topk_row if 0 <= int(b) < max_blocks}
    return np.asarray([j for j in range(int(abs_pos) + 1)
                       if j // SPARSE_BLOCK_SIZE in blocks], dtype=np.int64)


# ---------------------------------------------------------------------------
# O3. Exact decoding of stored codes
# ---------------------------------------------------------------------------

def bf16_value(bits):
    """bfloat16 bit patterns -> float64: the top half of an IEEE binary32."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return bits.view(np.float32).astype(np.float64)


def fp8_e4m3fn_value(code):
    """OCP FP8 E4M3FN code -> float64 (reading: the fn flavour, max 448).

    [FI] MiniMaxM3SparseFlashInferImpl.forward views the cache as the fp8
    dtype; the per-tensor scales are max|x| / 448, the E4M3FN maximum.
    Sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
    subnormal (2^-6 * m/8); S.1111.111 is NaN; there is no infinity.
    """
    code = np.asarray(code, dtype=np.int64)
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e2m1_value(nib):
    """OCP FP4 E2M1 code -> float64: sign bit, 2 exponent bits (bias 1), 1
    mantissa bit; exponent 0 is subnormal (m/2).  [NV4] stores K and V as
    packed e2m1 data plus block scales (customize_spec)."""
    nib = np.asarray(nib, dtype=np.int64)
    s = (nib >> 3) & 1
    e = (nib >> 1) & 3
    m = nib & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, e - 1))
    return np.where(s == 1, -mag, mag)


def nvfp4_token_values(slot_bytes, token, head_dim, global_scale, side="k"):
    """Decode tokens of NVFP4 (page, head-slot) byte rows -> [..., head_dim] fp64.

    ``slot_bytes`` [..., 9 * head_dim] uint8 are whole slots and ``token``
    [...] the token (0..15) to read from each; ``side`` says whether the slot
    is a K slot ("k") or a V slot ("v").
    [NV4] customize_spec: each head's K and V are two slots of packed data
    plus block scales; the bytes inside a page are laid out for the kernels.
    Reading (our layout; two e2m1 codes per byte, the low nibble holding the
    even element; value = e2m1 * E4M3FN scale of the element's group of 16 *
    global):
      K slot, token-major: token t's code byte c (elements 2c, 2c+1) at
        t*head_dim/2 + c; its scale of group u at 8*head_dim + t*head_dim/16 + u.
      V slot, in groups of 4 tokens: code byte c of token t at
        ((t//4 * head_dim/8 + c//4) * 4 + t%4) * 4 + c%4  (so the 4-byte units of
        the 4 tokens of a group that hold the same 8 elements are adjacent);
        its scale of group u at 8*head_dim + (t//4 * head_dim/16 + u) * 4 + t%4.
    PARITY UNPINNED for the byte order (a convention of ours; the kernels and
    the oracle follow the same written layout).
    """
    raw = np.asarray(slot_bytes, dtype=np.int64)
    t = np.asarray(token, dtype=np.int64)[..., None]
    d = np.arange(head_dim)
    c = d // 2                      # code byte of element d
    u = d // 16                     # its scale group
    if side == "k":
        code_at = t * (head_dim // 2) + c
        scale_at = PAGE_SIZE * (head_dim // 2) + t * (head_dim // 16) + u
    elif side == "v":
        code_at = ((t // 4 * (head_dim // 8) + c // 4) * 4 + t % 4) * 4 + c % 4
        scale_at = PAGE_SIZE * (head_dim // 2) + (t // 4 * (head_dim // 16) + u) * 4 + t % 4
    else:
        raise ValueError(side)
    byte = np.take_along_axis(raw, code_at, axis=-1)
    nib = np.where(d % 2 == 0, byte & 0xF, byte >> 4)
    scl = np.take_along_axis(raw, scale_at, axis=-1)
    return e2m1_value(nib) * fp8_e4m3fn_value(scl) * global_scale


# ---------------------------------------------------------------------------
# The paged cache, read by plain indexing
# ---------------------------------------------------------------------------

class PagedKVCache:
    """A paged K/V cache held as raw codes in numpy arrays.

    kv_dtype "bf16" / "fp8": k_pages and v_pages are [pages, Hkv, 16, D] of
    uint16 (bf16 bits) / uint8 (E4M3FN codes); ``k_scale`` / ``v_scale`` are
    the per-tensor dequant multipliers ([FI] MiniMaxM3SparseFlashInferImpl.
    forward folds them into the softmax scale and the output).
    kv_dtype "nvfp4": k_pages is [pages, 2*Hkv, 9*D] uint8, slot 2g = K and
    slot 2g+1 = V of kv head g ([NV4] customize_spec: two slots per head);
    ``k_scale`` / ``v_scale`` are the per-tensor global scales (reading: a
    multiplier in the same sense as the fp8 scale).

    ``block_page_stride`` ([SPA] minimax_m3_sparse_block_page_stride) is 8
    when K and V are separate planes and 16 when a block holds both sides;
    reading: then V of page p is page p + 8 of the V buffer ("reached from
    the same page id at a fixed offset").

    ``layout="rows128"`` (bf16 / fp8): k_pages is the one dense
    [pages, Hkv, 128, 2 * D] array of [FI] MiniMaxM3SparseFlashInferBackend.
    supported_kv_cache_layouts, each token row holding K then V; v_pages is
    unused.  Reading: page b is sparse block b and page-16 id
    b * block_page_stride + j names its rows 16 j .. 16 j + 15.
    """

    def __init__(self, kv_dtype, k_pages, v_pages, num_kv_heads, head_dim,
                 block_page_stride=PAGES_PER_SPARSE_BLOCK, k_scale=1.0, v_scale=1.0, layout="page16"):
        if kv_dtype not in ("bf16", "fp8", "nvfp4"):
            raise ValueError(kv_dtype)
        if layout not in ("page16", "rows128") or (layout == "rows128" and kv_dtype == "nvfp4"):
            raise ValueError(layout)
        self.layout = layout
        self.kv_dtype = kv_dtype
        self.k_pages = k_pages
        self.v_pages = v_pages
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.block_page_stride = block_page_stride
        self.k_scale = float(k_scale)
        self.v_scale = float(v_scale)

    def read_tokens(self, side, pages, slots):
        """Dequantized [n, Hkv, D] K ("k") or V ("v") of tokens at (page, slot)."""
        pages = np.asarray(pages, dtype=np.int64)
        slots = np.asarray(slots, dtype=np.int64)
        if self.kv_dtype == "nvfp4":
            heads = 2 * np.arange(self.num_kv_heads) + (0 if side == "k" else 1)
            raw = self.k_pages[pages[:, None], heads[None, :]]        # [n, Hkv, 9D]
            g = self.k_scale if side == "k" else self.v_scale
            tok = np.broadcast_to(slots[:, None], raw.shape[:2])
            return nvfp4_token_values(raw, tok, self.head_dim, g, side)
        if self.layout == "rows128":
            D = self.head_dim
            blk, j = pages // self.block_page_stride, pages % self.block_page_stride
            row = self.k_pages[blk, :, PAGE_SIZE * j + slots, :]              # [n, Hkv, 2D]
            raw = row[..., :D] if side == "k" else row[..., D:]
            scale = self.k_scale if side == "k" else self.v_scale
        elif side == "k":
            raw, scale = self.k_pages[pages, :, slots, :], self.k_scale
        else:
            off = self.block_page_stride - PAGES_PER_SPARSE_BLOCK
            raw, scale = self.v_pages[pages + off, :, slots, :], self.v_scale
        if self.kv_dtype == "bf16":
            return bf16_value(raw) * scale
        return fp8_e4m3fn_value(raw) * scale


def gather_tokens(cache, bt_row, token_ids):
    """K and V ([n, Hkv, D] fp64) of a request's logical tokens.

    Token j lives in logical block j // 128, whose physical block id is
    bt_row[j // 128] ([SPA] _write_sparse_block_table_row_from_values calls
    the looked-up value logical_page); its page-16 id is
    physical * block_page_stride + (j % 128) // 16 and its slot j % 16.
    """
    j = np.asarray(token_ids, dtype=np.int64)
    phys = np.asarray(bt_row, dtype=np.int64)[j // SPARSE_BLOCK_SIZE]
    pages = phys * cache.block_page_stride + (j % SPARSE_BLOCK_SIZE) // PAGE_SIZE
    slots = j % PAGE_SIZE
    return cache.read_tokens("k", pages, slots), cache.read_tokens("v", pages, slots)


# ---------------------------------------------------------------------------
# O4. Softmax attention over the mask
# ---------------------------------------------------------------------------

def attend_row(q_row, K, V, softmax_scale):
    """Softmax attention of one query row over the tokens it sees, fp64.

    q_row [Hq, D]; K, V [n, Hkv, D].  Reading (grouped-query attention, the
    pages do not print the mapping): q head h reads kv head h // (Hq / Hkv),
    torch's enable_gqa convention.  An empty context gives a zero output
    (reading: nothing to average).  PARITY UNPINNED for that zero: the pages
    print no output for an empty context, so it is a convention (the kernels
    follow the same one).
    """
    Hq, D = q_row.shape
    n, Hkv, _ = K.shape
    out = np.zeros((Hq, D))
    if n == 0:
        return out
    group = Hq // Hkv
    for g in range(Hkv):
        qg = q_row[g * group:(g + 1) * group]                  # heads of kv head g
        s = softmax_scale * (qg @ K[:, g, :].T)                 # [group, n]
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[g * group:(g + 1) * group] = (p / p.sum(axis=1, keepdims=True)) @ V[:, g, :]
    return out


def sparse_attention(q, cache, topk, block_table, req, abs_pos, softmax_scale, rows=None):
    """Outputs [len(rows), Hq, D] fp64 of the given rows (all rows by default).

    q [rows_total, Hq, D] (fp64 values of the bf16 input, layout of
    [FI] forward: query viewed as [tokens, num_heads, head_size]); the row's
    tokens come from the explicit mask (O2), their K/V from the paged cache
    by plain indexing, then fp64 softmax attention (O4).
    """
    if rows is None:
        rows = range(len(req))
    max_blocks = block_table.shape[1]
    outs = []
    for i in rows:
        toks = token_mask(topk[i], int(abs_pos[i]), max_blocks)
        if len(toks) == 0:
            outs.append(np.zeros(q.shape[1:]))
            continue
        K, V = gather_tokens(cache, block_table[int(req[i])], toks)
        outs.append(attend_row(np.asarray(q[i], dtype=np.float64), K, V, softmax_scale))
    return np.stack(outs) if outs else np.zeros((0,) + q.shape[1:])


# ---------------------------------------------------------------------------
# Index-cache insert
# ---------------------------------------------------------------------------

def insert_index_cache(index_k, index_cache, slot_mapping):
    """Scatter index keys into the key-only side cache, in place.

    [SPA] minimax_m3_insert_index_cache: keys [N, D] go into a cache
    [B, T, D], one int64 slot per key; nothing happens on empty
    input.  The kernel body is not printed; reading: slot s addresses block
    s // T, position s % T (the usual vLLM slot numbering), and negative
    slots (padding) are skipped.
    """
    if index_k.size == 0 or index_cache.size == 0:
        return index_cache
    T = index_cache.shape[1]
    for i in range(index_k.shape[0]):
        s = int(slot_mapping[i])
        if s < 0:
            continue
        index_cache[s // T, s % T, :] = index_k[i, :]
    return index_cache

