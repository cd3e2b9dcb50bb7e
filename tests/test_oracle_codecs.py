"""Pins of the oracle's number-format helpers against library casts.

The FP8 format (OCP E4M3FN, largest finite value 448) is the reading of
"V lowered to FP8" in the SageAttention deployment guide (pwwt.cn), sec. 1.
torch's float8_e4m3fn / float16 / bfloat16 casts are independent library
routines that round to nearest even.
"""
import numpy as np
import pytest
import torch

import oracle


def _all_fp16_values():
    bits = np.arange(65536, dtype=np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    return x[np.isfinite(x)]


def test_e4m3_encode_exhaustive_over_fp16():
    x = _all_fp16_values()
    xc = np.clip(x, -448.0, 448.0).astype(np.float32)
    ours = oracle.e4m3_encode(xc)
    ref = torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # every code agrees bit for bit, including the sign of zero (-0.0 -> 0x80)
    assert np.array_equal(ours, ref)
    assert ours[np.nonzero((xc == 0) & np.signbit(xc))[0][0]] == 0x80


def test_e4m3_encode_clamps_out_of_range():
    x = np.array([449.0, 464.0, 1e6, -500.0, -1e30], dtype=np.float32)
    codes = oracle.e4m3_encode(x)
    assert list(codes) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


@pytest.mark.parametrize("dtype,tdt", [("fp16", torch.float16), ("bf16", torch.bfloat16)])
def test_round_half_matches_torch(dtype, tdt):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-5).astype(np.float32),   # subnormal range of fp16
        (rng.standard_normal(5000) * 300).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26], dtype=np.float32),
    ])
    ours = oracle.round_half(x, dtype)
    ref = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)
