"""Pins for the oracle's codecs and quantiser (CPU only).

Each test checks the oracle against something other than itself: the
published code tables (tests/golden), PyTorch's own float8 conversions, a
scalar brute-force nearest-value search, and exact round trips.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mx

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_e2m1_table():
    rows = _rows("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = mx.decode_e2m1(int(code, 16))
        assert got == float(val) and np.signbit(got) == val.startswith("-"), (code, got)


def test_e4m3_anchors():
    for code, val in _rows("e4m3_anchors.txt"):
        got = float(mx.decode_e4m3(int(code, 16)))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), (code, got)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = mx.decode_e4m3(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e8m0_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = mx.decode_e8m0(codes)
    assert math.isnan(got[255]) and math.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])


def test_rne_golden_cases():
    for fmt, a, want in _rows("rne_cases.txt"):
        got = float(mx.round_to_grid(np.array(float(a)), fmt))
        assert got == float(want), (fmt, a, got, want)


@pytest.mark.parametrize("fmt,ncodes", [(mx.FMT_E4M3, 256), (mx.FMT_E2M1, 16)])
def test_encode_roundtrip_every_code(fmt, ncodes):
    codes = np.arange(ncodes, dtype=np.uint8)
    vals = mx.decode_e4m3(codes) if fmt == mx.FMT_E4M3 else mx.decode_e2m1(codes)
    ok = ~np.isnan(vals)
    back = mx.encode(vals[ok], fmt)
    np.testing.assert_array_equal(back, codes[ok])


def test_e4m3_encode_matches_torch_in_range():
    # torch's float32 -> float8_e4m3fn conversion rounds to nearest even; inside
    # the finite range (|v| <= 448) it must agree code for code, sign included.
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.6, 20000),
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, -2.0 ** -10, 1e-12, -1e-12]),
    ]).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = mx.encode(v.astype(np.float64), mx.FMT_E4M3)
    np.testing.assert_array_equal(got, ref)


def _nearest_even_bruteforce(a, table, mant_lsb):
    """Scalar nearest-value search over the positive grid, ties to the code with
    an even mantissa, saturating above the top of the grid."""
    if a >= table[-1]:
        return len(table) - 1
    best, bestd = None, None
    for c, t in enumerate(table):
        d = abs(a - t)
        if bestd is None or d < bestd or (d == bestd and mant_lsb(c) == 0):
            best, bestd = c, d
    return best


def _scalar_quantize_block(vals, fmt):
    """A second, loop-based MX quantiser written from the OCP rule with the
    math module: shared exponent from frexp, elements by brute-force search."""
    emax = 8 if fmt == mx.FMT_E4M3 else 2
    amax = max(abs(v) for v in vals)
    if amax == 0:
        E = -127
    else:
        _, e = math.frexp(amax)
        E = max(-127, min(127, (e - 1) - emax))
    if fmt == mx.FMT_E4M3:
        table = [float(mx.decode_e4m3(c)) for c in range(0x7F)]
        sign = 0x80
    else:
        table = [float(mx.decode_e2m1(c)) for c in range(8)]
        sign = 0x08
    codes = []
    for v in vals:
        c = _nearest_even_bruteforce(abs(v) / 2.0 ** E, table, lambda c: c & 1)
        codes.append(c | (sign if math.copysign(1.0, v) < 0 else 0))
    return codes, E + 127


@pytest.mark.parametrize("fmt", [mx.FMT_E4M3, mx.FMT_E2M1])
def test_quantize_mx_matches_scalar_bruteforce(fmt):
    rng = np.random.default_rng(11)
    rows = []
    for i in range(24):
        blk = rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 6)
        if i == 0:
            blk[:] = 0.0
        if i == 1:
            blk[:] = 0.0
            blk[5] = -3.0e-39          # far below 2^-127 * grid: scale code 0
        if i == 2:
            blk = np.round(blk)        # many exact ties after scaling
        rows.append(blk)
    v = np.stack(rows)
    q, s = mx.quantize_mx(v, fmt)
    codes = mx.unpack_fp4(q) if fmt == mx.FMT_E2M1 else q
    for i, blk in enumerate(rows):
        want_codes, want_scale = _scalar_quantize_block(list(blk), fmt)
        assert s[i, 0] == want_scale, (i, s[i, 0], want_scale)
        np.testing.assert_array_equal(codes[i], np.array(want_codes, dtype=np.uint8), err_msg=str(i))


def test_quantize_scale_bounds_and_dequant_error():
    # The OCP rule puts amax / 2^E in [2^emax, 2^(emax+1)); relative error of
    # an unsaturated element is at most half a grid step (2^-4 for E4M3).
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 256))
    q, s = mx.quantize_mx(v, mx.FMT_E4M3)
    d = mx.dequantize_mx(q, s, mx.FMT_E4M3)
    blocks = np.abs(v).reshape(64, 8, 32).max(-1)
    ratio = blocks / mx.decode_e8m0(s)
    assert np.all((ratio >= 256) & (ratio < 512))
    unsat = np.abs(v) / np.repeat(mx.decode_e8m0(s), 32, -1) <= 448
    rel = np.abs(d - v)[unsat & (np.abs(v) > 2.0 ** -6 * np.repeat(mx.decode_e8m0(s), 32, -1))] / \
        np.abs(v)[unsat & (np.abs(v) > 2.0 ** -6 * np.repeat(mx.decode_e8m0(s), 32, -1))]
    assert rel.max() <= 2.0 ** -4


def test_ceil_rule_never_saturates():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((32, 128)) * 100
    q, s = mx.quantize_mx(v, mx.FMT_E4M3, rule="ceil")
    ratio = np.abs(v).reshape(32, 4, 32).max(-1) / mx.decode_e8m0(s)
    assert np.all((ratio > 224) & (ratio <= 448))


def test_fp4_pack_order():
    codes = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    p = mx.pack_fp4(codes)
    np.testing.assert_array_equal(p, np.array([[0x21, 0x43]], dtype=np.uint8))
    np.testing.assert_array_equal(mx.unpack_fp4(p), codes)


def test_bf16_golden_cases():
    for a, want in _rows("bf16_cases.txt"):
        got = int(mx.bf16_rne(np.array(float(a))))
        assert got == int(want, 16), (a, hex(got), want)


def test_bf16_matches_torch_for_fp32_inputs():
    # From fp32 there is no double rounding, so torch's RNE conversion must agree.
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-30, 30, 50000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = mx.bf16_rne(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(mx.bf16_value(got), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())
