"""Workload recipes and seeded generators.

Every random draw of the metadata comes from numpy's PCG64 seeded with the
workload's seed; the large tensors (queries, K/V) come from a torch generator
seeded with the same number on the device they are built on.

Recipe (the five named workloads, plus reduced variants for tests):

* requests: sequence lengths fixed or uniform integers in [lo, hi];
  prefill requests carry new tokens after an optional context;
* block_table: every request needs ceil(seq / 128) physical 128-token blocks;
  all of them are drawn as one seeded permutation of the pool, so a request's
  blocks are scattered across the cache; unused columns hold block 0;
* top-k rows (one per query token, shared by all heads): the token's own block
  plus distinct uniformly chosen earlier blocks (as many as fit, up to k - 1),
  -1 for the remaining slots, the whole row shuffled; padded prefill rows get
  random in-range ids, which the method must drop;
* queries and K/V: N(0, 1) fp32, rounded to bf16 (RNE) or encoded to fp8
  E4M3FN with per-tensor scale max|x| / 448, or NVFP4 (e2m1 codes, one E4M3FN
  scale per 16 elements, per-tensor fp32 global scale max|x| / (6 * 448));
* only tokens that exist (position < seq_len) of blocks that some row selects
  are written; every other byte of the cache is 0xFF, which is NaN in all three
  formats, so a stray read shows up in the output.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = [
    "Workload", "CONFIGS", "make_workload", "make_query", "make_kv_cache",
    "encode_fp8_e4m3fn", "encode_nvfp4_rows", "arrange_nvfp4_slot", "NAN_BYTE",
    "written_blocks", "rows128_cache",
]

BLOCK = 128          # tokens per sparse block
PAGE = 16            # tokens per page
PAGES_PER_BLOCK = BLOCK // PAGE
NAN_BYTE = 0xFF      # NaN as bf16 (0xFFFF), as E4M3FN (0xFF) and as an NVFP4 scale


@dataclasses.dataclass
class Workload:
    name: str
    mode: str                      # "decode" | "prefill"
    kv_dtype: str                  # "bf16" | "fp8" | "nvfp4"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    topk_k: int
    seq_lens: np.ndarray           # int32 [R], KV length including new tokens
    decode_query_len: int          # decode only (1 for prefill)
    cu_seqlens_q: np.ndarray | None  # int32 [R + 1], prefill only
    total_q: int                   # rows, padded rows included
    block_table: np.ndarray        # int32 [R, max_blocks]
    num_phys_blocks: int
    topk: np.ndarray               # int32 [total_q, k]
    softmax_scale: float
    block_page_stride: int
    seed: int
    # the position each row was generated for (used only to draw its own block)
    gen_row_req: np.ndarray = dataclasses.field(repr=False, default=None)
    gen_row_pos: np.ndarray = dataclasses.field(repr=False, default=None)

    @property
    def num_reqs(self):
        return len(self.seq_lens)


# name -> recipe.  C1..C5 are the five named workloads; the *s variants are
# reduced copies (same heads / dims / k / dtype) that the CPU oracle finishes in
# seconds while still spanning several blocks, splits and a ragged tail.
CONFIGS = {
    "C1": dict(mode="decode", kv_dtype="bf16", seq_lens=[1000, 700], dql=1,
               Hq=4, Hkv=1, D=64, k=4, seed=1),
    "C2": dict(mode="decode", kv_dtype="bf16", num_reqs=64, seq_range=(4096, 32768), dql=1,
               Hq=64, Hkv=8, D=128, k=16, seed=2),
    "C3": dict(mode="decode", kv_dtype="fp8", num_reqs=32, seq_range=(8192, 65536), dql=4,
               Hq=64, Hkv=8, D=128, k=32, seed=3),
    "C4": dict(mode="prefill", kv_dtype="bf16", qlens=[2048, 4096, 8192, 8192], context=[0, 0, 0, 0],
               pad_rows=64, Hq=64, Hkv=8, D=128, k=16, seed=4),
    "C5": dict(mode="decode", kv_dtype="nvfp4", num_reqs=128, seq_range=(32768, 131072), dql=1,
               Hq=64, Hkv=8, D=128, k=32, seed=5),
    # reduced variants
    "C2s": dict(mode="decode", kv_dtype="bf16", num_reqs=3, seq_range=(200, 3000), dql=1,
                Hq=64, Hkv=8, D=128, k=16, seed=12),
    "C3s": dict(mode="decode", kv_dtype="fp8", num_reqs=2, seq_range=(500, 5000), dql=4,
                Hq=64, Hkv=8, D=128, k=32, seed=13),
    "C4s": dict(mode="prefill", kv_dtype="bf16", qlens=[300, 517], context=[0, 200],
                pad_rows=5, Hq=64, Hkv=8, D=128, k=16, seed=14),
    "C5s": dict(mode="decode", kv_dtype="nvfp4", num_reqs=2, seq_range=(1000, 6000), dql=1,
                Hq=64, Hkv=8, D=128, k=32, seed=15),
}


def _draw_row(rng, own_blk, k):
    """Own block plus up to k - 1 distinct earlier blocks, -1 padded, shuffled."""
    n_early = min(k - 1, own_blk)
    early = rng.choice(own_blk, size=n_early, replace=False) if n_early > 0 else np.zeros(0, np.int64)
    row = np.full(k, -1, dtype=np.int64)
    row[0] = own_blk
    row[1:1 + n_early] = early
    rng.shuffle(row)
    return row


def make_workload(name, *, block_page_stride=8, seed=None, selection="independent", **overrides):
    """Build the metadata of a named workload (numpy, seeded).

    selection: "independent" (every row draws its own earlier blocks, the
    named workloads) or "per_block" (the rows of a request whose positions
    share a 128-token block share one draw; a variant for measurement only,
    with the same context lengths)."""
    if selection not in ("independent", "per_block"):
        raise ValueError(f"selection {selection!r}")
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    seed = cfg["seed"] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    k = cfg["k"]
    if cfg["mode"] == "decode":
        if "seq_lens" in cfg:
            seq = np.asarray(cfg["seq_lens"], dtype=np.int64)
        else:
            lo, hi = cfg["seq_range"]
            seq = rng.integers(lo, hi + 1, size=cfg["num_reqs"])
        dql = cfg["dql"]
        cu = None
        total_q = len(seq) * dql
        row_req = np.repeat(np.arange(len(seq)), dql)
        row_pos = seq[row_req] - dql + np.tile(np.arange(dql), len(seq))
        n_real = total_q
    else:
        qlens = np.asarray(cfg["qlens"], dtype=np.int64)
        ctx = np.asarray(cfg["context"], dtype=np.int64)
        seq = qlens + ctx
        dql = 1
        cu = np.concatenate([[0], np.cumsum(qlens)])
        n_real = int(cu[-1])
        total_q = n_real + cfg["pad_rows"]
        row_req = np.concatenate([np.full(q, r) for r, q in enumerate(qlens)] + [np.zeros(cfg["pad_rows"], np.int64)])
        row_pos = np.concatenate([ctx[r] + np.arange(q) for r, q in enumerate(qlens)] + [np.full(cfg["pad_rows"], -1)])
    nblk = (seq + BLOCK - 1) // BLOCK
    pool = int(nblk.sum())
    perm = rng.permutation(pool)
    max_blocks = int(nblk.max())
    bt = np.zeros((len(seq), max_blocks), dtype=np.int64)
    off = 0
    for r, n in enumerate(nblk):
        bt[r, :n] = perm[off:off + n]
        off += n
    topk = np.full((total_q, k), -1, dtype=np.int64)
    shared = {}
    for i in range(total_q):
        if i < n_real and selection == "per_block":
            key = (int(row_req[i]), int(row_pos[i]) // BLOCK)
            if key not in shared:
                shared[key] = _draw_row(rng, key[1], k)
            topk[i] = shared[key]
        elif i < n_real:
            topk[i] = _draw_row(rng, int(row_pos[i]) // BLOCK, k)
        else:
            topk[i] = rng.choice(max_blocks, size=min(k, max_blocks), replace=False).tolist() + [-1] * (k - min(k, max_blocks))
    return Workload(
        name=name, mode=cfg["mode"], kv_dtype=cfg["kv_dtype"],
        num_q_heads=cfg["Hq"], num_kv_heads=cfg["Hkv"], head_dim=cfg["D"], topk_k=k,
        seq_lens=seq.astype(np.int32), decode_query_len=dql,
        cu_seqlens_q=None if cu is None else cu.astype(np.int32),
        total_q=int(total_q), block_table=bt.astype(np.int32), num_phys_blocks=pool,
        topk=topk.astype(np.int32), softmax_scale=1.0 / math.sqrt(cfg["D"]),
        block_page_stride=block_page_stride, seed=seed,
        gen_row_req=row_req, gen_row_pos=row_pos,
    )


def written_blocks(wl):
    """(request, logical block, tokens present) of every block some real row selects."""
    seen = {}
    for i in range(wl.total_q):
        if wl.gen_row_pos[i] < 0:
            continue
        r = int(wl.gen_row_req[i])
        nb = (int(wl.seq_lens[r]) + BLOCK - 1) // BLOCK
        for b in wl.topk[i]:
            b = int(b)
            if 0 <= b < nb and (r, b) not in seen:
                seen[(r, b)] = min(BLOCK, int(wl.seq_lens[r]) - BLOCK * b)
    return [(r, b, n) for (r, b), n in sorted(seen.items())]


def make_query(wl, device="cpu"):
    """q [total_q, Hq, D] bf16, N(0, 1) rounded to nearest even."""
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000 + 1)
    q = torch.randn((wl.total_q, wl.num_q_heads, wl.head_dim), generator=g, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16)


def encode_fp8_e4m3fn(x, scale):
    """x / scale clamped to +-448, rounded to nearest even E4M3FN, as uint8 codes."""
    y = (x / scale).clamp(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


_E2M1_EDGES = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e2m1_codes(y):
    """Round-to-nearest-even e2m1 codes of y (already clamped to +-6)."""
    a = y.abs()
    idx = torch.zeros_like(a, dtype=torch.int32)
    for n, edge in enumerate(_E2M1_EDGES):
        # ties go to the even code index: strict for odd n, inclusive for even n
        idx += (a >= edge).int() if n % 2 == 1 else (a > edge).int()
    sign = (y < 0).int() << 3
    return (idx | sign).to(torch.uint8)


def encode_nvfp4_rows(x, global_scale):
    """Encode rows x [..., D] -> (codes [..., D/2] uint8, scales [..., D/16] uint8).

    Each group of 16 consecutive elements gets the E4M3FN scale
    RNE(amax16 / (6 * global)); elements become RNE e2m1 codes of
    x / (scale * global); byte c holds element 2c in its low nibble.
    """
    *lead, D = x.shape
    g = x.reshape(*lead, D // 16, 16)
    amax = g.abs().amax(dim=-1)
    s_code = (amax / (6.0 * global_scale)).clamp(max=448.0).to(torch.float8_e4m3fn)
    s_val = s_code.to(torch.float32)
    denom = (s_val * global_scale).unsqueeze(-1)
    y = torch.where(denom > 0, g / torch.where(denom > 0, denom, torch.ones_like(denom)), torch.zeros_like(g))
    codes = _e2m1_codes(y.clamp(-6.0, 6.0)).reshape(*lead, D)
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed, s_code.view(torch.uint8)


def arrange_nvfp4_slot(codes, scales, v_side):
    """Bytes of NVFP4 slots from per-token codes [..., 16, D/2] and scales [..., 16, D/16].

    K slots are token-major: the 16 tokens' code bytes, then their scale
    bytes.  V slots group the tokens by 4 so that a decode lane finds the
    8-element code units of 4 tokens, and their 4 scales, adjacent: codes as
    [4 token groups][D/8 units of 4 bytes][4 tokens][4 bytes], then scales as
    [4 token groups][D/16 scale groups][4 tokens].
    """
    *lead, T, half = codes.shape
    D = 2 * half
    if v_side:
        codes = codes.reshape(*lead, T // 4, 4, D // 8, 4).transpose(-3, -2)
        scales = scales.reshape(*lead, T // 4, 4, D // 16).transpose(-2, -1)
    return torch.cat([codes.reshape(*lead, -1), scales.reshape(*lead, -1)], dim=-1)


def _f32(x):
    """Round a python float to the nearest fp32 value (scales are fp32 scalars)."""
    return float(np.float32(x))


def make_kv_cache(wl, device="cpu"):
    """Allocate and fill the paged cache of a workload.

    Returns a dict with ``k_pages`` / ``v_pages`` (uint8 byte tensors in the
    library's layout), ``k_scale`` / ``v_scale`` (python floats),
    ``page_stride_bytes`` and ``num_pages``.  bf16 / fp8: two planes
    [pages, Hkv, 16, D] (or one buffer holding both sides when
    block_page_stride is 16: K at 16b + j, V at 16b + 8 + j).  NVFP4: one
    buffer [pages, 2 * Hkv, 9 * D] (slot 2g = K, 2g + 1 = V; per slot the
    16 tokens' packed codes, then their scales, arranged by
    arrange_nvfp4_slot).
    """
    Hkv, D = wl.num_kv_heads, wl.head_dim
    stride = wl.block_page_stride
    num_pages = wl.num_phys_blocks * stride
    wb = written_blocks(wl)
    nb = len(wb)
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed * 1000 + 2)
    K = torch.randn((nb, BLOCK, Hkv, D), generator=gen, device=device, dtype=torch.float32)
    V = torch.randn((nb, BLOCK, Hkv, D), generator=gen, device=device, dtype=torch.float32)
    n_tok = torch.tensor([n for (_, _, n) in wb], dtype=torch.int64, device=device)
    present = torch.arange(BLOCK, device=device)[None, :] < n_tok[:, None]
    phys = torch.tensor([int(wl.block_table[r, b]) for (r, b, _) in wb], dtype=torch.int64, device=device)
    pm = present[:, :, None, None]
    k_scale = v_scale = 1.0
    if wl.kv_dtype == "bf16":
        esize = 2
        Kc = K.to(torch.bfloat16).view(torch.uint8).reshape(nb, BLOCK, Hkv, D * 2)
        Vc = V.to(torch.bfloat16).view(torch.uint8).reshape(nb, BLOCK, Hkv, D * 2)
    elif wl.kv_dtype == "fp8":
        esize = 1
        k_scale = _f32(float(K.abs().amax(dim=(2, 3))[present].max()) / 448.0) if nb else 1.0
        v_scale = _f32(float(V.abs().amax(dim=(2, 3))[present].max()) / 448.0) if nb else 1.0
        Kc = encode_fp8_e4m3fn(K, k_scale)
        Vc = encode_fp8_e4m3fn(V, v_scale)
    else:
        k_scale = _f32(float(K.abs().amax(dim=(2, 3))[present].max()) / (6.0 * 448.0)) if nb else 1.0
        v_scale = _f32(float(V.abs().amax(dim=(2, 3))[present].max()) / (6.0 * 448.0)) if nb else 1.0
        kd, ks = encode_nvfp4_rows(K, k_scale)
        vd, vs = encode_nvfp4_rows(V, v_scale)
    if wl.kv_dtype in ("bf16", "fp8"):
        row = D * esize
        page_bytes = Hkv * PAGE * row
        Kc = torch.where(pm, Kc, torch.full_like(Kc, NAN_BYTE))
        Vc = torch.where(pm, Vc, torch.full_like(Vc, NAN_BYTE))
        # [nb, 8 pages, 16, Hkv, row] -> [nb, 8, Hkv, 16, row]
        Kp = Kc.reshape(nb, PAGES_PER_BLOCK, PAGE, Hkv, row).permute(0, 1, 3, 2, 4).reshape(nb, PAGES_PER_BLOCK, page_bytes)
        Vp = Vc.reshape(nb, PAGES_PER_BLOCK, PAGE, Hkv, row).permute(0, 1, 3, 2, 4).reshape(nb, PAGES_PER_BLOCK, page_bytes)
        j = torch.arange(PAGES_PER_BLOCK, device=device)
        kidx = (phys[:, None] * stride + j[None, :]).reshape(-1)
        if stride == PAGES_PER_BLOCK:
            k_pages = torch.full((num_pages, page_bytes), NAN_BYTE, dtype=torch.uint8, device=device)
            v_pages = torch.full((num_pages, page_bytes), NAN_BYTE, dtype=torch.uint8, device=device)
            k_pages[kidx] = Kp.reshape(-1, page_bytes)
            v_pages[kidx] = Vp.reshape(-1, page_bytes)
        else:
            k_pages = torch.full((num_pages, page_bytes), NAN_BYTE, dtype=torch.uint8, device=device)
            v_pages = k_pages
            k_pages[kidx] = Kp.reshape(-1, page_bytes)
            k_pages[kidx + PAGES_PER_BLOCK] = Vp.reshape(-1, page_bytes)
        k_pages = k_pages.view(num_pages, Hkv, PAGE, row)
        v_pages = v_pages.view(num_pages, Hkv, PAGE, row)
    else:
        slot_bytes = PAGE * (D // 2) + PAGE * (D // 16)
        page_bytes = 2 * Hkv * slot_bytes

        def slots(dat, scl, v_side):
            dat = torch.where(pm, dat, torch.full_like(dat, NAN_BYTE))
            scl = torch.where(pm, scl, torch.full_like(scl, NAN_BYTE))
            # [nb, 128, Hkv, *] -> [nb, 8 pages, Hkv, 16 tokens, *]
            dat = dat.reshape(nb, PAGES_PER_BLOCK, PAGE, Hkv, D // 2).permute(0, 1, 3, 2, 4)
            scl = scl.reshape(nb, PAGES_PER_BLOCK, PAGE, Hkv, D // 16).permute(0, 1, 3, 2, 4)
            return arrange_nvfp4_slot(dat, scl, v_side)   # [nb, 8, Hkv, slot_bytes]

        both = torch.stack([slots(kd, ks, False), slots(vd, vs, True)], dim=3)  # [nb, 8, Hkv, 2, slot]
        j = torch.arange(PAGES_PER_BLOCK, device=device)
        kidx = (phys[:, None] * stride + j[None, :]).reshape(-1)
        k_pages = torch.full((num_pages, page_bytes), NAN_BYTE, dtype=torch.uint8, device=device)
        k_pages[kidx] = both.reshape(-1, page_bytes)
        k_pages = k_pages.view(num_pages, 2 * Hkv, slot_bytes)
        v_pages = None
    return dict(k_pages=k_pages, v_pages=v_pages, k_scale=k_scale, v_scale=v_scale,
                page_stride_bytes=page_bytes, num_pages=num_pages, layout="page16")


def rows128_cache(cache, wl, layers=1, layer=0):
    """The same bf16 / fp8 cache re-laid as 128-token pages with K|V rows.

    Page b (= sparse block b) is [Hkv, 128 tokens, K row bytes then V row
    bytes]; with ``layers`` > 1 the pages sit in a block-outer buffer, page b
    of this layer at (b * layers + layer) * page bytes, the other layers'
    bytes NaN-filled.  Needs a cache of block_page_stride 8.  Returns a dict
    like make_kv_cache's: ``k_pages`` [blocks, Hkv, 128, 2 * row] uint8,
    ``v_pages`` None, ``layout`` "rows128".
    """
    if wl.kv_dtype not in ("bf16", "fp8") or wl.block_page_stride != PAGES_PER_BLOCK:
        raise ValueError("rows128 holds bf16 / fp8 caches of block_page_stride 8")
    k, v = cache["k_pages"], cache["v_pages"]
    n16, Hkv, _, row = k.shape
    nb = n16 // PAGES_PER_BLOCK

    def per_block(t):   # [n16, Hkv, 16, row] -> [nb, Hkv, 128, row]
        return t.reshape(nb, PAGES_PER_BLOCK, Hkv, PAGE, row).permute(0, 2, 1, 3, 4).reshape(nb, Hkv, BLOCK, row)

    rows = torch.cat([per_block(k), per_block(v)], dim=-1)           # [nb, Hkv, 128, 2 row]
    page_bytes = Hkv * BLOCK * 2 * row
    big = torch.full((nb, layers, page_bytes), NAN_BYTE, dtype=torch.uint8, device=k.device)
    big[:, layer] = rows.reshape(nb, page_bytes)
    pages = big[:, layer].view(nb, Hkv, BLOCK, 2 * row)
    out = dict(cache)
    out.update(k_pages=pages, v_pages=None, page_stride_bytes=layers * page_bytes, num_pages=nb,
               layout="rows128")
    return out
