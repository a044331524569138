"""Pins of the MXFP8 quantiser oracle (OCP MX v1.0, MXFP8 E4M3: one E8M0 scale
per 32 values, X = floor(log2(max |v|)) - 8).

What fixes it from outside the oracle:
* the E4M3 value of every code equals torch's float8_e4m3fn decoding;
* every element code equals torch's float8_e4m3fn cast (round to nearest even)
  of v / 2^X wherever |v / 2^X| <= 448 (torch does not saturate beyond);
* the shared exponent satisfies its definition 2^(X+8) <= max|v| < 2^(X+9);
* closed cases: exactly representable blocks round-trip, ties go to the even
  code (normal and subnormal), values past 448 saturate, zero blocks, sign
  symmetry, and the error bound of a 3-bit significand.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3(y):
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy(), t.float().numpy().astype(np.float64)


def test_code_values_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.nanmax(got) == 448.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def random_blocks(n, seed):
    rng = np.random.default_rng(seed)
    # bf16 values of widely varying magnitude, with a few exact zeros
    mag = np.exp2(rng.integers(-20, 20, size=(n, 1)))
    x = rng.normal(size=(n, 32)) * mag
    x[rng.random((n, 32)) < 0.02] = 0.0
    x32 = x.astype(np.float32)
    bf = (x32.view(np.uint32) & 0xFFFF0000).view(np.float32)  # truncate to bf16: exact in f32 and f64
    return bf.astype(np.float64)


@pytest.mark.parametrize("seed", range(3))
def test_shared_exponent_definition_and_codes_match_torch(seed):
    x = random_blocks(2000, seed)
    codes, scales = oracle.quantize_mxfp8(x)
    X = scales.astype(np.int64)[:, 0] - 127
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    assert (np.exp2(X[nz] + 8) <= amax[nz]).all() and (amax[nz] < np.exp2(X[nz] + 9)).all()
    assert (X[~nz] == -127).all()
    y = x / np.exp2(X)[:, None]
    inside = np.abs(y) <= 448
    tc, tv = torch_e4m3(y)
    assert (codes[inside] == tc[inside]).all()
    assert (codes[~inside] & 0x7F == 0x7E).all()  # beyond 448: saturated
    deq = oracle.dequantize_mxfp8(codes, scales)
    np.testing.assert_array_equal(deq[inside], tv[inside] * np.exp2(X)[:, None].repeat(32, 1)[inside])


def test_representable_blocks_round_trip_exactly():
    rng = np.random.default_rng(4)
    finite = [c for c in range(0x7F)]
    vals = np.array([oracle.e4m3_value(c) for c in finite])
    for k in (-20, -3, 0, 5, 17):
        blk = rng.choice(vals, size=32) * rng.choice([-1.0, 1.0], size=32)
        blk[0] = 448.0  # sets the shared exponent to k
        x = blk * 2.0 ** k
        np.testing.assert_array_equal(oracle.mxfp8_roundtrip(x), x)


def test_ties_go_to_the_even_code():
    x = np.zeros(32)
    x[0] = 300.0          # X = 0
    x[1] = 1.0625         # between 1.0 (m=0) and 1.125 (m=1): to 1.0
    x[2] = 1.1875         # between 1.125 (m=1) and 1.25 (m=2): to 1.25
    x[3] = 1.5 * 2 ** -9  # subnormal tie between codes 1 and 2: to code 2
    x[4] = 0.5 * 2 ** -9  # tie between 0 and code 1: to 0
    x[5] = 2.5 * 2 ** -9  # tie between codes 2 and 3: to code 2
    x[6] = -1.0625
    got = oracle.mxfp8_roundtrip(x)
    np.testing.assert_array_equal(got[1:7], [1.0, 1.25, 2 * 2 ** -9, 0.0, 2 * 2 ** -9, -1.0])


def test_saturation_and_zero_blocks():
    x = np.zeros((2, 32))
    x[0, 0] = 511.0   # X = 0: 511 saturates
    x[0, 1] = 464.0   # the midpoint to the (absent) 480 saturates too
    x[0, 2] = -460.0
    codes, scales = oracle.quantize_mxfp8(x)
    assert scales[0, 0] == 127 and scales[1, 0] == 0
    assert list(codes[0, :3]) == [0x7E, 0x7E, 0xFE]
    assert (codes[1] == 0).all()
    np.testing.assert_array_equal(oracle.dequantize_mxfp8(codes, scales)[1], 0.0)


@pytest.mark.parametrize("seed", range(2))
def test_sign_symmetry_and_error_bound(seed):
    x = random_blocks(1000, 10 + seed)
    c1, s1 = oracle.quantize_mxfp8(x)
    c2, s2 = oracle.quantize_mxfp8(-x)
    np.testing.assert_array_equal(s1, s2)
    nz = x != 0
    assert ((c1 ^ c2)[nz] == 0x80).all()
    X = s1.astype(np.int64)[:, :1] - 127
    y = np.abs(x) / np.exp2(X)
    err = np.abs(oracle.dequantize_mxfp8(c1, s1) - x) / np.exp2(X)
    # half a unit in the last place: 2^(e-4) for normal y (e = floor(log2 y) >= -6), 2^-10 below
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    bound = np.where(y >= 2.0 ** -6, 2.0 ** (e - 4), 2.0 ** -10)
    inside = y <= 448
    assert (err[inside] <= bound[inside]).all()
    # past 448 (the block's top values, y < 512) the value saturates to 448
    assert (y < 512).all() and (err[~inside] == (y[~inside] - 448)).all()


def test_rows_of_several_blocks_are_independent():
    x = random_blocks(8, 20).reshape(2, 128)
    codes, scales = oracle.quantize_mxfp8(x)
    assert codes.shape == (2, 128) and scales.shape == (2, 4)
    for b in range(4):
        c, s = oracle.quantize_mxfp8(x[:, 32 * b:32 * b + 32])
        np.testing.assert_array_equal(codes[:, 32 * b:32 * b + 32], c)
        np.testing.assert_array_equal(scales[:, b:b + 1], s)
