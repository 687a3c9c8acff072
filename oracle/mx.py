"""Exact codecs for the microscaled (MX) element and scale formats, fp64.

Test infrastructure only (see the package header): nothing in the product
path may import this module.

The layer quantises activations to FP8 E4M3 and weights to FP4 E2M1 or FP8
E4M3, each block of 32 consecutive K-elements sharing one E8M0 power-of-two
scale (GC-MoE summary page, "Approach" and "Limitations": FP8 x FP4 grouped
GEMM, the "(1,1,32)" scale recipe; fusion-kernel blog, "Fusing MXFP8/NVFP4
quantisation" section). The pages fix the formats by name only; the bit
layouts and the conversion rule below follow the OCP Microscaling Formats
(MX) v1.0 specification:

* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; no inf/NaN.
* E4M3 ("fn" variant): sign bit 7, exponent bits 6..3 (bias 7), mantissa
  bits 2..0; exponent 0 is subnormal; S.1111.111 is NaN; max finite 448.
* E8M0: an unsigned biased exponent, value 2^(c-127); 0xFF is NaN.
* MX block quantisation: shared exponent E = floor(log2(amax)) - emax_elem,
  clamped to [-127, 127] (emax_elem = 8 for E4M3, 2 for E2M1); each element
  is v / 2^E rounded to nearest, ties to even, saturated to the largest
  finite magnitude. amax = 0 (or below 2^-127) gives scale code 0.

Two packing conventions are this library's own: FP4 codes are packed two to a
byte with element 2i in the low nibble, and a rounded value of either sign
keeps the sign bit of its input (so a negative value that rounds to zero is
encoded as negative zero).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
FMT_E2M1 = "e2m1"
FMT_E4M3 = "e4m3"

E4M3_MAX = 448.0
E2M1_MAX = 6.0
_EMAX = {FMT_E4M3: 8, FMT_E2M1: 2}
_MANT_BITS = {FMT_E4M3: 3, FMT_E2M1: 1}
_MIN_EXP = {FMT_E4M3: -6, FMT_E2M1: 0}      # exponent of the smallest normal
_MAXV = {FMT_E4M3: E4M3_MAX, FMT_E2M1: E2M1_MAX}
_SIGN = {FMT_E4M3: 0x80, FMT_E2M1: 0x08}


# ---------------------------------------------------------------- decoding
def decode_e2m1(codes) -> np.ndarray:
    """E2M1 code (0..15, one per array element) -> exact fp64 value."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int32)))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_e4m3(codes) -> np.ndarray:
    """E4M3 (fn) code byte -> exact fp64 value; 0x7F and 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0,
                   np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_e8m0(codes) -> np.ndarray:
    """E8M0 scale byte -> 2^(c-127) in fp64; 0xFF decodes to NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    v = np.ldexp(1.0, (c - 127).astype(np.int32))
    return np.where(c == 255, np.nan, v)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] E2M1 codes; element 2i is the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """[..., K] E2M1 codes -> [..., K/2] bytes; element 2i is the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return ((c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def dequantize_mx(q: np.ndarray, s: np.ndarray, fmt: str) -> np.ndarray:
    """Element codes + E8M0 block scales (one per 32 along the last axis) -> fp64.

    For E2M1, `q` is packed (two codes per byte). The product of an element and
    a power-of-two scale is exact in fp64 for every finite code pair.
    """
    codes = unpack_fp4(q) if fmt == FMT_E2M1 else np.asarray(q, dtype=np.uint8)
    K = codes.shape[-1]
    assert K % BLOCK == 0 and s.shape[-1] == K // BLOCK, (codes.shape, s.shape)
    vals = decode_e2m1(codes) if fmt == FMT_E2M1 else decode_e4m3(codes)
    scale = np.repeat(decode_e8m0(s), BLOCK, axis=-1)
    return vals * scale


# -------------------------------------------------------------- rounding
def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for finite a > 0, exact (via frexp, not log2)."""
    _, e = np.frexp(a)
    return e.astype(np.int64) - 1


def round_to_grid(a: np.ndarray, fmt: str) -> np.ndarray:
    """Round non-negative fp64 magnitudes to the nearest element of the format's
    grid, ties to even, saturating at the largest finite magnitude."""
    a = np.asarray(a, dtype=np.float64)
    assert np.all(a >= 0) and np.all(np.isfinite(a))
    mb = _MANT_BITS[fmt]
    with np.errstate(divide="ignore"):
        e = np.where(a > 0, _floor_log2(np.where(a > 0, a, 1.0)), _MIN_EXP[fmt])
    e = np.maximum(e, _MIN_EXP[fmt])
    quantum = np.ldexp(1.0, (e - mb).astype(np.int32))
    r = np.rint(a / quantum) * quantum          # np.rint: round half to even
    return np.minimum(r, _MAXV[fmt])


def _positive_table(fmt: str) -> np.ndarray:
    if fmt == FMT_E2M1:
        return decode_e2m1(np.arange(8))
    return decode_e4m3(np.arange(0x7F))         # 0x00..0x7E, increasing


def encode(v: np.ndarray, fmt: str) -> np.ndarray:
    """Round fp64 values (already divided by their block scale) to element
    codes: RNE, saturating, sign bit taken from the input's sign bit."""
    v = np.asarray(v, dtype=np.float64)
    r = round_to_grid(np.abs(v), fmt)
    table = _positive_table(fmt)
    code = np.searchsorted(table, r)
    assert np.all(table[np.minimum(code, len(table) - 1)] == r), "value off the grid"
    code = code.astype(np.uint8)
    return np.where(np.signbit(v), code | _SIGN[fmt], code).astype(np.uint8)


def block_scale_exponent(amax: np.ndarray, fmt: str, rule: str = "ocp") -> np.ndarray:
    """Shared exponent E of a block (scale = 2^E) from its amax.

    rule "ocp":  E = clamp(floor(log2 amax) - emax_elem, -127, 127)
    rule "ceil": E = clamp(ceil(log2(amax / max_finite)), -127, 127)
    amax = 0 gives E = -127 under both rules.
    """
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    safe = np.where(pos, amax, 1.0)
    if rule == "ocp":
        E = _floor_log2(safe) - _EMAX[fmt]
    elif rule == "ceil":
        ratio = safe / _MAXV[fmt]
        fl = _floor_log2(ratio)
        exact = np.ldexp(1.0, fl.astype(np.int32)) == ratio
        E = np.where(exact, fl, fl + 1)
    else:
        raise ValueError(rule)
    E = np.where(pos, E, -127)
    return np.clip(E, -127, 127).astype(np.int64)


def quantize_mx(v: np.ndarray, fmt: str, rule: str = "ocp"):
    """Quantise along the last axis in blocks of 32.

    Returns (codes, scales): codes uint8 [..., K] for E4M3 or packed [..., K/2]
    for E2M1; scales uint8 E8M0 [..., K/32].
    """
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v)), "non-finite input to the quantiser"
    K = v.shape[-1]
    assert K % BLOCK == 0, K
    blocks = v.reshape(v.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    E = block_scale_exponent(amax, fmt, rule)
    scaled = blocks / np.ldexp(1.0, E.astype(np.int32))[..., None]   # exact: power of two
    codes = encode(scaled, fmt).reshape(v.shape)
    scales = (E + 127).astype(np.uint8)
    if fmt == FMT_E2M1:
        codes = pack_fp4(codes)
    return codes, scales


# ------------------------------------------------------------------ bf16
def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp64 -> bfloat16 bit patterns (uint16), one rounding, nearest-even.

    Rounds directly from fp64 (no intermediate fp32 rounding). Magnitudes at or
    above the rounding threshold past the largest finite bf16 become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x))
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.where(a > 0, _floor_log2(np.where(a > 0, a, 1.0)), -126)
    e = np.maximum(e, -126)                          # bf16 subnormals share 2^-126's quantum
    quantum = np.ldexp(1.0, (e - 7).astype(np.int32))
    r = np.rint(a / quantum) * quantum
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    signed = np.where(np.signbit(x), -r, r).astype(np.float32)   # exact: r is on the bf16 grid
    return (signed.view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
