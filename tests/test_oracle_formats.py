"""Pins of the oracle's number formats against torch's own casts (a library
the oracle does not use) and against closed forms of the formats.

e4m3 here is the OCP FP8 E4M3 format ("e4m3fn"): bias 7, 3 mantissa bits,
subnormals m * 2^-9, no infinity, NaN = 0x7F / 0xFF, largest finite 448.
bf16 is the upper half of IEEE binary32.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e4m3_encode(v32):
    t = torch.from_numpy(np.asarray(v32, dtype=np.float32).copy())
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits[np.isfinite(f)]


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(codes[nan].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_decode_closed_forms():
    d = oracle.e4m3_decode
    assert d([0x7E])[0] == 448.0
    assert d([0x01])[0] == 2.0 ** -9          # smallest subnormal
    assert d([0x07])[0] == 7 * 2.0 ** -9      # largest subnormal
    assert d([0x08])[0] == 2.0 ** -6          # smallest normal
    assert d([0x38])[0] == 1.0
    assert d([0xB8])[0] == -1.0
    v = d([0x80])[0]
    assert v == 0.0 and np.signbit(v)
    # values increase strictly with the code over 0x00..0x7E
    pos = d(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def test_e4m3_encode_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)],
                     dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


@pytest.mark.parametrize("scale", [1.0, 0.015625, 3.0 / 448.0, 0.37, 1e-3,
                                   7.25e-6])
def test_e4m3_encode_matches_torch_cast_on_all_bf16(scale):
    bits = all_finite_bf16()
    x = oracle.bf16_decode(bits)
    v = (x / np.float32(scale)).astype(np.float32)
    v = np.clip(v, np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    ours = oracle.e4m3_encode(v)
    ref = torch_e4m3_encode(v)
    assert np.array_equal(ours, ref)


def test_e4m3_encode_ties_and_signed_zero():
    # midpoints between neighbouring codes go to the even code
    enc = oracle.e4m3_encode
    assert enc([17.0])[0] == 0x58 and enc([19.0])[0] == 0x5A
    assert enc([2.0 ** -10])[0] == 0x00 and enc([3 * 2.0 ** -10])[0] == 0x02
    assert enc([-2.0 ** -11])[0] == 0x80
    assert enc([-0.0])[0] == 0x80
    # grid step in [256, 512) is 32: 384 (m=4), 416 (m=5), 448 (m=6)
    assert enc([432.0])[0] == 0x7E      # tie 416|448 -> 448 (even mantissa)
    assert enc([400.0])[0] == 0x7C      # tie 384|416 -> 384 (even mantissa)
    assert enc([424.0])[0] == 0x7D      # nearer 416
    assert enc([449.0])[0] == 0xFF      # outside the domain is rejected


def test_bf16_encode_matches_torch_cast():
    g = np.random.default_rng(123)
    u = g.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # force a quarter of them to exact ties, and some to near-max magnitudes
    u[::4] = (u[::4] & 0xFFFF0000) | 0x8000
    u[1::16] = (u[1::16] & 0x807FFFFF) | 0x7F000000
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.bf16_encode(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ours, ref.view(np.uint16))


def test_bf16_decode_is_upper_half():
    bits = all_finite_bf16()
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    assert np.array_equal(oracle.bf16_decode(bits), ref.to(torch.float32).numpy())
