"""Pins for the oracle's format decoding (CPU only).

The MXFP4 layout is the one of Mxfp4MoEMethod.create_weights on the vLLM
mxfp4 API page: packed e2m1 pairs along K and one e8m0 scale per 32.
"""
import math

import numpy as np
import pytest
import torch

from tests.decode_ref import (E2M1_TABLE, dequant_int4g32, dequant_mxfp4, e2m1_from_bits,
                              e8m0_torch, unpack_nibbles)


def test_e2m1_all_codes_closed_form(orc):
    for c in range(16):
        want = e2m1_from_bits(c)
        got = orc.e2m1_value(c)
        assert got == want, (c, got, want)
        assert math.copysign(1.0, got) == math.copysign(1.0, want), c  # -0 for code 8


def test_e2m1_value_set(orc):
    vals = sorted({abs(orc.e2m1_value(c)) for c in range(16)})
    assert vals == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e8m0_all_bytes_vs_torch(orc):
    ref = e8m0_torch(np.arange(256, dtype=np.uint8))
    for b in range(256):
        got = orc.e8m0_value(b)
        if b == 255:
            assert math.isnan(got) and math.isnan(ref[b])
        else:
            assert np.float32(got) == np.float32(ref[b]), b
            assert got == math.ldexp(1.0, b - 127)


def test_nibble_roundtrip_all_bytes(orc):
    row = np.arange(256, dtype=np.uint8)
    for b in range(256):
        assert orc.nibble(row, 2 * b) == (b & 0xF)
        assert orc.nibble(row, 2 * b + 1) == (b >> 4)
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=64, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    assert [orc.nibble(packed, k) for k in range(64)] == codes.tolist()
    assert np.array_equal(unpack_nibbles(packed), codes)


@pytest.mark.parametrize("v", [0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.0078125, 3.0e38,
                               3.4e38, -3.4e38, 1e-40, -1e-40, 2.0 ** -133, float("inf"),
                               float("-inf"), 0.0712890625, 6.0 / 7.0, 1.0 / 3.0])
def test_f32_to_bf16_rne_vs_torch(orc, v):
    want = int(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).view(torch.int16)[0]) & 0xFFFF
    assert orc.f32_to_bf16(v) == want


def test_f32_to_bf16_random_vs_torch(orc):
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.standard_normal(2000).astype(np.float32) * 100,
                           (rng.integers(0, 2**32, 2000, dtype=np.uint64)).astype(np.uint32).view(np.float32)])
    vals = vals[np.isfinite(vals)]
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)
    nan_bits = orc.f32_to_bf16(float("nan"))
    assert (nan_bits & 0x7F80) == 0x7F80 and (nan_bits & 0x7F) != 0


def test_dequant_mxfp4_vs_closed_form(orc):
    rng = np.random.default_rng(11)
    rows, K = 6, 128
    w = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    s = rng.integers(110, 140, size=(rows, K // 32), dtype=np.uint8)
    got = orc.dequant(w, s, orc.FMT_MXFP4, K)
    want = dequant_mxfp4(w, s)
    assert np.array_equal(got, want)
    # spot check one element by hand: row 3, k 37 -> byte 18 high nibble, block 1
    code = w[3, 18] >> 4
    assert got[3, 37] == E2M1_TABLE[code] * 2.0 ** (int(s[3, 1]) - 127)


def test_dequant_int4g32_vs_closed_form(orc):
    rng = np.random.default_rng(12)
    rows, K = 5, 96
    w = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    sf = rng.standard_normal((rows, K // 32)).astype(np.float32)
    s = torch.from_numpy(sf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.dequant(w, s, orc.FMT_INT4G32, K)
    want = dequant_int4g32(w, s)
    assert np.array_equal(got, want)
    # code 0x8 is -8, 0x7 is +7, 0xF is -1
    w1 = np.array([[0x78, 0xF0] * (K // 4)], dtype=np.uint8)
    one = torch.ones((1, K // 32), dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    d = orc.dequant(w1, one, orc.FMT_INT4G32, K)
    assert d[0, :4].tolist() == [-8.0, 7.0, 0.0, -1.0]
