"""MiniMax-M3 block-sparse attention over a paged KV cache, for MI355X (gfx950).

Thin ctypes binding over ``libmsa.so`` (C ABI in ``include/msa.h``).  Every
step of the computation runs in the library's HIP kernels; this module only
checks tensor dtypes / devices / shapes, passes raw device pointers and the
current HIP stream, and allocates outputs with torch when the caller gives
none.  There is no fallback: if the library is missing, every call raises.

Entry points (same names as the C ABI):

* ``msa_build_sparse_block_table`` - page-16 sparse table + context lengths
* ``msa_query_token_positions``    - prefill request ids and positions
* ``msa_sparse_decode``            - block-sparse GQA decode
* ``msa_sparse_decode_noalloc``    - the same decode with no workspace (library-held scratch)
* ``msa_sparse_prefill``           - block-sparse ragged causal prefill
* ``msa_insert_index_cache``       - index-key side-cache scatter
* ``msa_debug_gather_dequant``     - test hook: each row's K/V as an attend gathers them
"""

from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

__all__ = [
    "MsaError", "KVCache", "library_path", "load_library",
    "msa_build_sparse_block_table", "msa_query_token_positions",
    "msa_sparse_decode", "msa_sparse_decode_noalloc", "msa_sparse_prefill", "msa_sparse_attention", "msa_insert_index_cache",
    "msa_debug_gather_dequant", "msa_decode_workspace_size", "msa_prefill_workspace_size",
    "MSA_BF16", "MSA_FP16", "MSA_FP8_E4M3FN", "MSA_NVFP4", "MSA_FP32",
]

MSA_BF16, MSA_FP16, MSA_FP8_E4M3FN, MSA_NVFP4, MSA_FP32 = 0, 1, 2, 3, 4
_STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARGUMENT", 2: "MSA_ERR_UNSUPPORTED",
           3: "MSA_ERR_WORKSPACE_TOO_SMALL", 4: "MSA_ERR_HIP"}
_KV_DTYPES = {"bf16": MSA_BF16, "fp8": MSA_FP8_E4M3FN, "nvfp4": MSA_NVFP4}
_KV_LAYOUTS = {"page16": 0, "rows128": 1}


class MsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path():
    """The in-tree libmsa.so (MSA_LIBRARY names another build, e.g. the host
    sanitizer copy the CPU tests load)."""
    return os.environ.get("MSA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")


class _KV(ctypes.Structure):
    _fields_ = [
        ("kv_dtype", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_page_stride", ctypes.c_int32),
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("page_stride_bytes", ctypes.c_int64), ("num_pages", ctypes.c_int64),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("kv_layout", ctypes.c_int32),
    ]


_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "msa_last_error": ([], ctypes.c_char_p),
    "msa_build_sparse_block_table": ([_P, _I64, _I32, _I32, _P, _I64, _I32, _I32, _P, _I32, _P, _P, _I32,
                                      _P, _I64, _P, _P], _I32),
    "msa_query_token_positions": ([_P, _P, _I32, _I32, _P, _P, _P], _I32),
    "msa_decode_workspace_size": ([_I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_decode": ([_P, _I32, _I32, _I32, _I32, ctypes.POINTER(_KV), _P, _I64, _I32, _P, _I64, _I32,
                           _P, _F32, _P, _P, _SZ, _P], _I32),
    "msa_sparse_decode_noalloc": ([_P, _I32, _I32, _I32, _I32, ctypes.POINTER(_KV), _P, _I64, _I32, _P, _I64,
                                   _I32, _P, _F32, _P, _P], _I32),
    "msa_decode_noalloc_scratch_bytes": ([], _SZ),
    "msa_prefill_workspace_size": ([_I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_prefill": ([_P, _I32, _I32, _I32, ctypes.POINTER(_KV), _P, _I64, _I32, _P, _I64, _I32, _I32,
                            _P, _P, _F32, _P, _P, _SZ, _P], _I32),
    "msa_sparse_attention": ([_P, _I32, _I32, _I32, ctypes.POINTER(_KV), _P, _I64, _I32, _I32, _I32,
                              _P, _I64, _I32, _P, _I32, _P, _I64, _I32, _P, _P, _F32, _P, _P, _SZ, _P], _I32),
    "msa_insert_index_cache": ([_P, _I64, _I64, _I32, _I32, _I32, _P, _I64, _I64, _I64, _I32, _I32, _P, _I64,
                                _P], _I32),
    "msa_debug_gather_dequant": ([ctypes.POINTER(_KV), _P, _I64, _P, _I32, _I32, _I32, _P, _P, _P], _I32),
}
_lib = None


def load_library():
    """Load libmsa.so (built in-tree by ``block_sparse_paged_query_amd.build``)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python -m block_sparse_paged_query_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _call(name, *args):
    lib = load_library()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise MsaError(st, lib.msa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype=None, dim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D, got shape {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if device is not None and t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if t.dim() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} needs a contiguous last dimension")


def _need_table_rows(block_table, num_reqs, name):
    """The kernels read row r of the block table for every request r: a
    shorter table would be read past its end on the device."""
    if block_table.shape[0] < num_reqs:
        raise ValueError(f"{name} has {block_table.shape[0]} rows for {num_reqs} requests")


@dataclasses.dataclass
class KVCache:
    """One layer's paged K/V cache (layouts in include/msa.h).

    ``k_pages`` / ``v_pages``: tensors whose first dimension is the page (any
    dtype; bytes are what count).  ``k_scale`` / ``v_scale``: 1-element fp32
    device tensors or None (= 1.0).  ``layout``: "page16" (16-token pages, K
    and V planes or NVFP4 slots) or "rows128" (128-token pages
    [pages, Hkv, 128, 2 * D] with K|V-interleaved rows; ``v_pages`` None or
    the V view ``cache[..., D:]`` of the same tensor).
    """
    kv_dtype: str
    k_pages: torch.Tensor
    v_pages: torch.Tensor | None
    num_kv_heads: int
    head_dim: int
    block_page_stride: int = 8
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None
    layout: str = "page16"

    def _struct(self):
        if self.kv_dtype not in _KV_DTYPES:
            raise ValueError(f"kv_dtype {self.kv_dtype!r}: one of {sorted(_KV_DTYPES)}")
        if self.layout not in _KV_LAYOUTS:
            raise ValueError(f"layout {self.layout!r}: one of {sorted(_KV_LAYOUTS)}")
        kp = self.k_pages
        if self.layout == "page16" and kp.shape[0] > 0 and not kp[0].is_contiguous():
            raise ValueError("each page of k_pages must be dense in memory (only the page stride is free)")
        if self.layout == "page16" and self.v_pages is not None and self.v_pages.shape[0] > 0 \
                and not self.v_pages[0].is_contiguous():
            raise ValueError("each page of v_pages must be dense in memory (only the page stride is free)")
        if kp.device.type != "cuda":
            raise ValueError(f"k_pages must be a GPU tensor, got {kp.device}")
        if self.v_pages is not None and self.v_pages.device != kp.device:
            raise ValueError(f"v_pages is on {self.v_pages.device}, k_pages on {kp.device}")
        for name, s in (("k_scale", self.k_scale), ("v_scale", self.v_scale)):
            if s is not None:
                _need(s, name, torch.float32, device=kp.device)
                if s.numel() != 1:
                    raise ValueError(f"{name} must hold one element")
        stride = kp.stride(0) * kp.element_size()
        if self.v_pages is not None and self.kv_dtype != "nvfp4":
            if self.v_pages.stride(0) * self.v_pages.element_size() != stride:
                raise ValueError("k_pages and v_pages must share a page stride")
            if self.v_pages.shape[0] != kp.shape[0]:
                raise ValueError("k_pages and v_pages must hold the same number of pages")
        return _KV(_KV_DTYPES[self.kv_dtype], self.num_kv_heads, self.head_dim, self.block_page_stride,
                   kp.data_ptr(), None if self.v_pages is None else self.v_pages.data_ptr(),
                   stride, kp.shape[0],
                   None if self.k_scale is None else self.k_scale.data_ptr(),
                   None if self.v_scale is None else self.v_scale.data_ptr(),
                   _KV_LAYOUTS[self.layout])


def msa_build_sparse_block_table(topk, block_table, *, seq_lens=None, decode_query_len=1, query_req_id=None,
                                 query_abs_pos=None, block_page_stride=8, sparse_bt=None, sparse_ctx=None):
    """Page-16 sparse block table ([total_q, 8k] int32) and context lengths ([total_q] int32).

    Decode mode with ``seq_lens`` (rows = batch * decode_query_len), prefill
    mode with ``query_req_id`` and ``query_abs_pos``.  ``topk`` may be
    [total_q, k] or the pages' [1, total_q, k].
    """
    if topk.dim() == 3:
        topk = topk[0]
    if query_req_id is None:
        # decode mode: the kernel takes block_table's row count as the request
        # count and reads seq_lens[r] for each of them
        if seq_lens is None:
            raise ValueError("decode-mode tables need seq_lens (or query_req_id / query_abs_pos for prefill)")
        if seq_lens.shape[0] != block_table.shape[0]:
            raise ValueError(f"seq_lens has {seq_lens.shape[0]} requests, block_table {block_table.shape[0]} rows")
    dev = topk.device
    _need(topk, "topk", torch.int32, 2)
    _need(block_table, "block_table", torch.int32, 2, dev)
    total_q, k = topk.shape
    if sparse_bt is None:
        sparse_bt = torch.empty((total_q, 8 * k), dtype=torch.int32, device=dev)
    if sparse_ctx is None:
        sparse_ctx = torch.empty((total_q,), dtype=torch.int32, device=dev)
    _need(sparse_bt, "sparse_bt", torch.int32, 2, dev)
    _need(sparse_ctx, "sparse_ctx", torch.int32, 1, dev)
    if query_req_id is not None:
        _need(query_req_id, "query_req_id", torch.int32, 1, dev)
        _need(query_abs_pos, "query_abs_pos", torch.int32, 1, dev)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    _call("msa_build_sparse_block_table", _ptr(topk), topk.stride(0), k, total_q,
          _ptr(block_table), block_table.stride(0), block_table.shape[1], block_table.shape[0],
          _ptr(seq_lens), decode_query_len, _ptr(query_req_id), _ptr(query_abs_pos), block_page_stride,
          _ptr(sparse_bt), sparse_bt.stride(0), _ptr(sparse_ctx), _stream(dev))
    return sparse_bt, sparse_ctx


def msa_query_token_positions(cu_seqlens_q, context_lens, total_q):
    """Per-token request id and absolute position of a prefill batch (int32 pair)."""
    dev = cu_seqlens_q.device
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    req = torch.empty((total_q,), dtype=torch.int32, device=dev)
    pos = torch.empty((total_q,), dtype=torch.int32, device=dev)
    _call("msa_query_token_positions", _ptr(cu_seqlens_q), _ptr(context_lens), context_lens.shape[0], total_q,
          _ptr(req), _ptr(pos), _stream(dev))
    return req, pos


def msa_decode_workspace_size(total_q, num_q_heads, head_dim, topk_k):
    return load_library().msa_decode_workspace_size(total_q, num_q_heads, head_dim, topk_k)


def msa_prefill_workspace_size(total_q, num_q_heads, head_dim, topk_k):
    return load_library().msa_prefill_workspace_size(total_q, num_q_heads, head_dim, topk_k)


def _check_workspace(ws):
    # the library writes workspace_bytes bytes from the pointer on, on the GPU
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if ws.device.type != "cuda":
        raise ValueError(f"workspace must be a GPU tensor, got {ws.device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _ws_args(ws, device):
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    return _ptr(ws), ws.numel() * ws.element_size()


def _check_q(q, name="q"):
    _need(q, name, torch.bfloat16, 3)
    if q.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {q.device}")
    if not q.is_contiguous():
        raise ValueError(f"{name} must be contiguous [rows, heads, head_dim]")


def msa_sparse_decode(q, kv: KVCache, topk, block_table, seq_lens, softmax_scale, *, decode_query_len=1,
                      out=None, workspace=None):
    """Block-sparse GQA decode; q/out [batch * decode_query_len, Hq, D] bf16."""
    _check_workspace(workspace)
    if topk.dim() == 3:
        topk = topk[0]
    _need_table_rows(block_table, seq_lens.shape[0], "block_table")
    dev = q.device
    _check_q(q)
    _need(topk, "topk", torch.int32, 2, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_q(out, "out")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    rows, hq, d = q.shape
    if topk.shape[0] != rows:
        raise ValueError(f"topk has {topk.shape[0]} rows, q has {rows}")
    if d != kv.head_dim:
        raise ValueError(f"q head_dim {d} != cache head_dim {kv.head_dim}")
    num_reqs = seq_lens.shape[0]
    if rows != num_reqs * decode_query_len:
        raise ValueError(f"q has {rows} rows; {num_reqs} requests x decode_query_len {decode_query_len} "
                         f"= {num_reqs * decode_query_len}")
    if workspace is None:
        nbytes = msa_decode_workspace_size(rows, hq, d, topk.shape[1])
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _ws_args(workspace, dev)
    kvs = kv._struct()
    _call("msa_sparse_decode", _ptr(q), MSA_BF16, num_reqs, decode_query_len, hq, ctypes.byref(kvs),
          _ptr(topk), topk.stride(0), topk.shape[1], _ptr(block_table), block_table.stride(0),
          block_table.shape[1], _ptr(seq_lens), float(softmax_scale), _ptr(out), ws_ptr, ws_bytes, _stream(dev))
    return out


def msa_sparse_decode_noalloc(q, kv: KVCache, topk, block_table, seq_lens, softmax_scale, *, out,
                              decode_query_len=1):
    """msa_sparse_decode with no workspace: the library's own per-GPU scratch
    holds the split partials, and nothing is allocated (``out`` is required).
    Calls that overlap in time on one GPU share that scratch and race."""
    if topk.dim() == 3:
        topk = topk[0]
    _need_table_rows(block_table, seq_lens.shape[0], "block_table")
    dev = q.device
    _check_q(q)
    _check_q(out, "out")
    _need(topk, "topk", torch.int32, 2, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    if out.shape != q.shape or out.device != dev:
        raise ValueError("out must have q's shape and device")
    rows, hq, d = q.shape
    if topk.shape[0] != rows:
        raise ValueError(f"topk has {topk.shape[0]} rows, q has {rows}")
    if d != kv.head_dim:
        raise ValueError(f"q head_dim {d} != cache head_dim {kv.head_dim}")
    num_reqs = seq_lens.shape[0]
    if rows != num_reqs * decode_query_len:
        raise ValueError(f"q has {rows} rows; {num_reqs} requests x decode_query_len {decode_query_len} "
                         f"= {num_reqs * decode_query_len}")
    kvs = kv._struct()
    _call("msa_sparse_decode_noalloc", _ptr(q), MSA_BF16, num_reqs, decode_query_len, hq, ctypes.byref(kvs),
          _ptr(topk), topk.stride(0), topk.shape[1], _ptr(block_table), block_table.stride(0),
          block_table.shape[1], _ptr(seq_lens), float(softmax_scale), _ptr(out), _stream(dev))
    return out


def msa_sparse_prefill(q, kv: KVCache, topk, block_table, cu_seqlens_q, seq_lens, softmax_scale, *, out=None,
                       workspace=None):
    """Block-sparse ragged causal prefill; q/out [total_q, Hq, D] bf16 (padded rows -> 0)."""
    _check_workspace(workspace)
    if topk.dim() == 3:
        topk = topk[0]
    _need_table_rows(block_table, seq_lens.shape[0], "block_table")
    dev = q.device
    _check_q(q)
    _need(topk, "topk", torch.int32, 2, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_q(out, "out")
    total_q, hq, d = q.shape
    if topk.shape[0] != total_q:
        raise ValueError(f"topk has {topk.shape[0]} rows, q has {total_q}")
    if cu_seqlens_q.shape[0] != seq_lens.shape[0] + 1:
        raise ValueError("cu_seqlens_q must have num_reqs + 1 entries")
    if workspace is None:
        nbytes = msa_prefill_workspace_size(total_q, hq, d, topk.shape[1])
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _ws_args(workspace, dev)
    kvs = kv._struct()
    _call("msa_sparse_prefill", _ptr(q), MSA_BF16, total_q, hq, ctypes.byref(kvs), _ptr(topk), topk.stride(0),
          topk.shape[1], _ptr(block_table), block_table.stride(0), block_table.shape[1], seq_lens.shape[0],
          _ptr(cu_seqlens_q), _ptr(seq_lens), float(softmax_scale), _ptr(out), ws_ptr, ws_bytes, _stream(dev))
    return out


def msa_sparse_attention(q, kv: KVCache, topk, num_decode_tokens, softmax_scale, *, decode_block_table=None,
                         decode_seq_lens=None, decode_query_len=1, prefill_block_table=None,
                         prefill_cu_seqlens_q=None, prefill_seq_lens=None, out=None, workspace=None):
    """A whole batch: decode rows [0, num_decode_tokens), then prefill rows.

    q/out [num_tokens, Hq, D] bf16; topk [num_tokens, k] token-major.  The
    decode part uses decode_block_table / decode_seq_lens, the prefill part
    prefill_block_table / prefill_cu_seqlens_q (from the first prefill row) /
    prefill_seq_lens; a part with no rows needs none of its tensors.
    """
    _check_workspace(workspace)
    if topk.dim() == 3:
        topk = topk[0]
    nd = int(num_decode_tokens)
    if nd > 0 and decode_block_table is not None and decode_seq_lens is not None:
        _need_table_rows(decode_block_table, decode_seq_lens.shape[0], "decode_block_table")
    if nd < q.shape[0] and prefill_block_table is not None and prefill_seq_lens is not None:
        _need_table_rows(prefill_block_table, prefill_seq_lens.shape[0], "prefill_block_table")
    dev = q.device
    _check_q(q)
    _need(topk, "topk", torch.int32, 2, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_q(out, "out")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    num_tokens, hq, d = q.shape
    if topk.shape[0] != num_tokens:
        raise ValueError(f"topk has {topk.shape[0]} rows, q has {num_tokens}")
    if d != kv.head_dim:
        raise ValueError(f"q head_dim {d} != cache head_dim {kv.head_dim}")
    if not 0 <= nd <= num_tokens:
        raise ValueError(f"num_decode_tokens {nd} of {num_tokens} rows")
    dbt = dsl = pbt = pcu = psl = None
    if nd > 0:
        _need(decode_block_table, "decode_block_table", torch.int32, 2, dev)
        _need(decode_seq_lens, "decode_seq_lens", torch.int32, 1, dev)
        if nd != decode_seq_lens.shape[0] * decode_query_len:
            raise ValueError(f"{nd} decode rows; {decode_seq_lens.shape[0]} requests x decode_query_len "
                             f"{decode_query_len}")
        dbt, dsl = decode_block_table, decode_seq_lens
    if nd < num_tokens:
        _need(prefill_block_table, "prefill_block_table", torch.int32, 2, dev)
        _need(prefill_cu_seqlens_q, "prefill_cu_seqlens_q", torch.int32, 1, dev)
        _need(prefill_seq_lens, "prefill_seq_lens", torch.int32, 1, dev)
        if prefill_cu_seqlens_q.shape[0] != prefill_seq_lens.shape[0] + 1:
            raise ValueError("prefill_cu_seqlens_q must have num_prefill_reqs + 1 entries")
        pbt, pcu, psl = prefill_block_table, prefill_cu_seqlens_q, prefill_seq_lens
    if workspace is None:
        # the two parts run one after the other and reuse one workspace
        nbytes = max(msa_decode_workspace_size(max(nd, 1), hq, d, topk.shape[1]),
                     msa_prefill_workspace_size(num_tokens - nd, hq, d, topk.shape[1]))
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _ws_args(workspace, dev)
    kvs = kv._struct()
    _call("msa_sparse_attention", _ptr(q), MSA_BF16, num_tokens, hq, ctypes.byref(kvs), _ptr(topk), topk.stride(0),
          topk.shape[1], nd, decode_query_len,
          None if dbt is None else _ptr(dbt), 0 if dbt is None else dbt.stride(0), 0 if dbt is None else dbt.shape[1],
          None if dsl is None else _ptr(dsl),
          0 if psl is None else psl.shape[0],
          None if pbt is None else _ptr(pbt), 0 if pbt is None else pbt.stride(0), 0 if pbt is None else pbt.shape[1],
          None if pcu is None else _ptr(pcu), None if psl is None else _ptr(psl),
          float(softmax_scale), _ptr(out), ws_ptr, ws_bytes, _stream(dev))
    return out


_ELEM = {torch.bfloat16: MSA_BF16, torch.float16: MSA_FP16, torch.float32: MSA_FP32,
         torch.float8_e4m3fn: MSA_FP8_E4M3FN}


def msa_insert_index_cache(index_k, index_cache, index_slot_mapping):
    """Scatter index keys [N, D] into the key-only cache [B, T, D] by slot (in place).

    Nothing is done when either tensor is empty.  The three tensors share a
    GPU; keys and cache share one of bf16 / fp16 / fp32 / fp8 E4M3FN; the
    slots are int64, one per key; the cache's key dimension is contiguous.
    """
    if index_k.numel() == 0 or index_cache.numel() == 0:
        return
    _need(index_cache, "index_cache", dim=3)
    _need(index_k, "index_k", index_cache.dtype, 2)
    _need(index_slot_mapping, "index_slot_mapping", torch.int64, 1)
    if index_cache.dtype not in _ELEM:
        raise TypeError(f"index_cache dtype {index_cache.dtype}: bf16, fp16, fp32 or float8_e4m3fn")
    n, d = index_k.shape
    if d != index_cache.shape[2]:
        raise ValueError(f"index_k rows hold {d} elements, index_cache rows {index_cache.shape[2]}")
    if index_slot_mapping.shape[0] != n:
        raise ValueError(f"{index_slot_mapping.shape[0]} slots for {n} keys")
    dev = index_cache.device
    for t, name in ((index_cache, "index_cache"), (index_k, "index_k"), (index_slot_mapping, "index_slot_mapping")):
        _need(t, name, device=dev)
    _call("msa_insert_index_cache", _ptr(index_k), index_k.stride(0), index_k.stride(1), n, d,
          _ELEM[index_k.dtype], _ptr(index_cache), index_cache.stride(0), index_cache.stride(1),
          index_cache.stride(2), index_cache.shape[0], index_cache.shape[1], _ptr(index_slot_mapping),
          index_slot_mapping.stride(0), _stream(dev))


def msa_debug_gather_dequant(kv: KVCache, sparse_bt, sparse_ctx, path="decode"):
    """fp32 K and V ([rows, 16 * width, Hkv, D] each) of every row's tokens in
    sparse-table order, as the decode attend's gather (path "decode") or the
    prefill attend's staging (path "prefill") produces them."""
    dev = kv.k_pages.device
    _need(sparse_bt, "sparse_bt", torch.int32, 2, dev)
    _need(sparse_ctx, "sparse_ctx", torch.int32, 1, dev)
    if path not in ("decode", "prefill"):
        raise ValueError(f"path {path!r}: 'decode' or 'prefill'")
    rows, width = sparse_bt.shape
    if sparse_ctx.shape[0] != rows:
        raise ValueError(f"sparse_ctx has {sparse_ctx.shape[0]} rows, sparse_bt {rows}")
    k = torch.empty((rows, 16 * width, kv.num_kv_heads, kv.head_dim), dtype=torch.float32, device=dev)
    v = torch.empty_like(k)
    kvs = kv._struct()
    _call("msa_debug_gather_dequant", ctypes.byref(kvs), _ptr(sparse_bt), sparse_bt.stride(0), _ptr(sparse_ctx),
          rows, width, 0 if path == "decode" else 1, _ptr(k), _ptr(v), _stream(dev))
    return k, v
