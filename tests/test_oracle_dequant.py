"""Pins of the oracle's code decoding (CPU only).

fp8 and bf16 are checked exhaustively against torch's CPU casts (library
routines); e2m1 against the OCP MX specification's value table; the NVFP4 byte
layout against hand-placed bytes; the encoder/decoder pair against the format's
rounding bound.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import arrange_nvfp4_slot, encode_nvfp4_rows

# OCP Microscaling Formats v1.0, FP4 E2M1: codes 0..7 are these magnitudes,
# codes 8..15 their negatives.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_fp8_all_codes_match_torch():
    codes = np.arange(256)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.fp8_e4m3fn_value(codes)
    nan = np.isnan(ref)
    assert nan.tolist() == np.isnan(got).tolist()
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF]
    assert (got[~nan] == ref[~nan]).all()
    assert got[0x7E] == 448.0 and got[1] == 2.0 ** -9


def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_value(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()


def test_e2m1_codes_match_ocp_table():
    got = oracle.e2m1_value(np.arange(16))
    want = E2M1_TABLE + [-v for v in E2M1_TABLE]
    assert got.tolist() == want


def test_nvfp4_products_exact_in_half_types():
    # every (e2m1 code, E4M3FN scale) product is representable in bf16 and fp16:
    # the dequantized value loses nothing before the contraction
    e = oracle.e2m1_value(np.arange(16))[:, None]
    s = oracle.fp8_e4m3fn_value(np.arange(256))[None, :]
    prod = (e * s)[:, ~np.isnan(s[0])].ravel()
    for dt in (torch.bfloat16, torch.float16):
        back = torch.from_numpy(prod).to(dt).to(torch.float64).numpy()
        assert (back == prod).all()
    assert np.abs(prod).max() == 6 * 448


def test_nvfp4_byte_layout():
    # one (page, slot) of head_dim 128: 16 tokens x 64 code bytes, then 16 x 8 scales
    D = 128
    slot = np.zeros(9 * D, dtype=np.uint8)
    t, c = 5, 37                          # token 5, byte 37 -> elements 74 (low), 75 (high)
    slot[t * 64 + c] = 0x3A               # low nibble 0xA = -1.0, high nibble 0x3 = 1.5
    slot[16 * 64 + t * 8 + 74 // 16] = 0x40   # E4M3FN 0x40 = 2.0 for elements 64..79
    vals = oracle.nvfp4_token_values(np.stack([slot] * 16), np.arange(16), D, 0.5)
    assert vals.shape == (16, D)
    nz = np.argwhere(vals != 0)
    assert nz.tolist() == [[5, 74], [5, 75]]
    assert vals[5, 74] == -1.0 * 2.0 * 0.5 and vals[5, 75] == 1.5 * 2.0 * 0.5


@pytest.mark.parametrize("side", ["k", "v"])
def test_nvfp4_slot_order_matches_the_generator(side):
    # The oracle reads slots by index arithmetic; the generator writes them by
    # tensor reshapes and transposes.  Random codes and scales, arranged by the
    # generator, must decode to e2m1(code) * scale read from the unarranged
    # per-token arrays.
    g = torch.Generator().manual_seed(11)
    codes = torch.randint(0, 256, (3, 16, 64), generator=g, dtype=torch.uint8)
    scales = torch.randint(0, 127, (3, 16, 8), generator=g, dtype=torch.uint8)   # finite E4M3FN
    slots = arrange_nvfp4_slot(codes, scales, side == "v").numpy()
    assert slots.shape == (3, 9 * 128)
    d = np.arange(128)
    for s in range(3):
        got = oracle.nvfp4_token_values(np.stack([slots[s]] * 16), np.arange(16), 128, 0.25, side)
        c = codes[s].numpy()[:, d // 2].astype(np.int64)
        nib = np.where(d % 2 == 0, c & 0xF, c >> 4)
        sc = oracle.fp8_e4m3fn_value(scales[s].numpy()[:, d // 16].astype(np.int64))
        assert np.array_equal(got, oracle.e2m1_value(nib) * sc * 0.25)


def test_nvfp4_encode_decode_within_rounding_bound():
    # the generator's encoder and the oracle's decoder are independent codes of
    # the same format: the round trip errs by at most half an e2m1 step at the
    # element's magnitude (1 between 4 and 6, 0.5 between 2 and 4, ...) times
    # the block scale, plus the scale's own rounding when the block max
    # rounds up (then |x| / scale < 6 and RNE stays within the same bound).
    g = torch.Generator().manual_seed(0)
    x = torch.randn(64, 128, generator=g)
    glob = float(x.abs().max()) / (6 * 448)
    data, scales = encode_nvfp4_rows(x, glob)
    slot = np.zeros((64, 9 * 128), dtype=np.uint8)
    # place row i as token 0 of its own slot
    slot[:, :64] = data.numpy()
    slot[:, 16 * 64:16 * 64 + 8] = scales.numpy()
    dec = oracle.nvfp4_token_values(slot, np.zeros(64, dtype=np.int64), 128, glob)
    s = oracle.fp8_e4m3fn_value(scales.numpy().astype(np.int64))      # [64, 8]
    step = np.repeat(s, 16, axis=1) * glob                              # block scale per element
    y = np.abs(x.numpy()) / step                                        # magnitude in e2m1 units
    half_ulp = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    err = np.abs(dec - x.numpy()) / step
    assert (err <= half_ulp + 1e-6).all()
    # and the data is not degenerate: most codes are nonzero
    assert (dec != 0).mean() > 0.8
