"""Pins for the oracle's small-float conversions (e4m3, binary16, bfloat16).

Each conversion is checked against something other than the oracle itself:
the format's printed grid points (tests/golden/e4m3_points.txt), and the
independent library conversions of torch (float8_e4m3fn, bfloat16) and numpy
(float16), all round-to-nearest-even.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def _f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def _near(vals32):
    """Values, their fp32 neighbours one ulp away, and both signs."""
    v = np.asarray(vals32, np.float32)
    up = np.nextafter(v, np.float32(np.inf))
    dn = np.nextafter(v, np.float32(-np.inf))
    allv = np.concatenate([v, up, dn])
    return np.concatenate([allv, -allv])


# ---- e4m3 -------------------------------------------------------------------

def test_e4m3_golden_points():
    for code, val in read_golden("e4m3_points.txt"):
        c = int(code, 16)
        got = oracle.e4m3_decode(np.array([c], np.uint8))[0]
        assert got == float(val), (code, got, val)
        if c not in (0x7F, 0xFF):
            assert np.signbit(got) == val.startswith("-"), code


def test_e4m3_decode_matches_torch_all_codes():
    c = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(c)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.where(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert np.all(ours[nan] == 0.0)  # S.1111.111 reads back as 0


def test_e4m3_encode_roundtrip_all_codes():
    c = np.array([i for i in range(256) if i not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(c).astype(np.float32)
    back = oracle.e4m3_encode(vals)
    np.testing.assert_array_equal(back, c)


def test_e4m3_encode_matches_torch_at_midpoints_and_random():
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448 ascending
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact in fp32
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)
    rng = np.random.default_rng(7)
    rnd = np.concatenate([
        rng.uniform(-448, 448, 200000),
        rng.standard_normal(200000) * 2.0 ** rng.integers(-14, 8, 200000),
    ]).astype(np.float32)
    x = np.concatenate([_near(mids), _near(pos.astype(np.float32)), rnd])
    x = x[np.abs(x) <= 448]
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.where(ours != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(ours[i]), hex(ref[i])) for i in bad[:8]]


def test_e4m3_ties_go_to_even_mantissa():
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    codes = oracle.e4m3_encode(mids)
    assert np.all(codes % 2 == 0)
    assert np.all((codes == np.arange(0, 0x7E)) | (codes == np.arange(1, 0x7F)))


def test_e4m3_saturates_and_keeps_sign_of_zero():
    x = np.array([448.0, 449.0, 1e30, np.inf, -470.0, -1e-30, 1e-30, 2.0 ** -10, -(2.0 ** -10)], np.float32)
    got = oracle.e4m3_encode(x)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x00, 0x80]
    # 2^-10 is the midpoint between 0 and the smallest subnormal 2^-9: ties to even (0).
    assert oracle.e4m3_encode(np.array([np.nextafter(np.float32(2 ** -10), np.float32(1))], np.float32))[0] == 1


# ---- binary16 ----------------------------------------------------------------

def test_f16_matches_numpy_dense_sweep():
    h = np.arange(0x7C00, dtype=np.uint16)
    vals = h.view(np.float16).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact: 12 significant bits
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32)
    rnd = _f32(bits)
    rnd = rnd[np.isfinite(rnd)]
    x = np.concatenate([_near(mids), _near(vals.astype(np.float32)), rnd,
                        np.array([65504, 65519.99, 65520, 65536, 1e9, -65520], np.float32)])
    ours = oracle.f16_encode(x)
    ref = x.astype(np.float16).view(np.uint16)
    bad = np.where(ours != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(ours[i]), hex(ref[i])) for i in bad[:8]]


def test_f16_decode_matches_numpy_all_finite():
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    ours = oracle.f16_decode(h)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])
    assert np.all(np.isinf(ours[np.isinf(ref)]))


def test_f16_from_double_matches_numpy():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100000) * 2.0 ** rng.integers(-30, 17, 100000)
    ours = oracle.f16_encode(x.astype(np.float64))
    ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


# ---- bfloat16 ----------------------------------------------------------------

def test_bf16_matches_torch():
    rng = np.random.default_rng(5)
    b = rng.integers(0, 0x7F80, 20000).astype(np.uint16)
    v = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nxt = ((b.astype(np.uint32) + 1) << 16).view(np.float32).astype(np.float64)
    mids = ((v + nxt) / 2).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    rnd = _f32(bits)
    rnd = rnd[np.isfinite(rnd)]
    x = np.concatenate([_near(mids), rnd])
    ours = oracle.bf16_encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.where(ours != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(ours[i]), hex(ref[i])) for i in bad[:8]]
