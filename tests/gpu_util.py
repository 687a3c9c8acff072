"""Helpers for the GPU parity tests: device upload of oracle-made inputs and
the comparison rules. Imported only by tests marked `gpu`."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import mx

DEV = "cuda"


def banner(msg: str) -> None:
    """Name the case before each GPU step so a failing run says which it was."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return host(t).view(np.uint16)


# ------------------------------------------------------------------ rules
def e4m3_ulp(mag_scaled: np.ndarray) -> np.ndarray:
    """Grid spacing of E4M3 at a scaled magnitude (value / block scale)."""
    m = np.maximum(mag_scaled, 2.0 ** -6)
    e = np.floor(np.log2(m))
    return np.ldexp(1.0, (e - 3).astype(np.int32))


# Bound on the GPU's fp32 dot-product error relative to the sum of |terms|,
# for the data these tests use (MX-quantised Gaussian draws and the h they
# produce):
#  - the fp32 accumulator takes one rounding per 128-wide K-tile and one per
#    level of the K-split tree (at most K/128 + 5 roundings of at most 2^-24 of
#    a partial sum each): 3.6e-6 at the largest K here (7168);
#  - inside one scaled MFMA the 128 products are not summed like an IEEE fp32
#    FMA chain. Measured by these tests (the largest error left after the two
#    BF16 roundings and the propagated input differences, over every element):
#    1.4e-6 to 6.4e-6 of the sum of |terms| on the decode and full-expert
#    shapes, 1.49e-5 on the 16K-token prefill's W2 (MXFP8 h x MXFP8 weights,
#    whose E4M3 blocks span a wide range); random full-range FP8 bytes, which
#    no test feeds, reach 2.6e-4.
# 2^-14 (6.1e-5) is four times the largest measured.
MFMA_REL = 2.0 ** -14


def assert_mx_within_1ulp(q_gpu, s_gpu, q_ref, s_ref, what: str, max_frac_diff: float = 0.02,
                          extra_tol=None):
    """FP8 requantised values may differ by at most one E4M3 step at the
    coarser of the two block scales (plus `extra_tol`, the propagated bound of
    the fp32 accumulation, where given); report how many codes/scales differ."""
    q_gpu, s_gpu = np.asarray(q_gpu), np.asarray(s_gpu)
    q_ref, s_ref = np.asarray(q_ref), np.asarray(s_ref)
    assert q_gpu.shape == q_ref.shape and s_gpu.shape == s_ref.shape, (what, q_gpu.shape, q_ref.shape)
    a = mx.dequantize_mx(q_gpu, s_gpu, mx.FMT_E4M3)
    b = mx.dequantize_mx(q_ref, s_ref, mx.FMT_E4M3)
    X = np.repeat(np.maximum(mx.decode_e8m0(s_gpu), mx.decode_e8m0(s_ref)), 32, axis=-1)
    tol = e4m3_ulp(np.maximum(np.abs(a), np.abs(b)) / X) * X
    if extra_tol is not None:
        tol = tol + extra_tol
    diff = np.abs(a - b)
    bad = diff > tol * (1 + 1e-12)
    frac_q = float(np.mean(q_gpu != q_ref)) if q_gpu.size else 0.0
    frac_s = float(np.mean(s_gpu != s_ref)) if s_gpu.size else 0.0
    worst = float(np.max(diff / np.maximum(tol, 1e-300))) if diff.size else 0.0
    print(f"  {what}: codes differing {frac_q:.2e}, scales differing {frac_s:.2e}, "
          f"beyond 1 ulp {int(bad.sum())}, largest |diff| / tolerance {worst:.3f}", flush=True)
    assert not bad.any(), f"{what}: {int(bad.sum())} values beyond 1 E4M3 ulp"
    assert frac_q <= max_frac_diff, f"{what}: {frac_q:.3f} of codes differ"


def _bf16_ulp(v):
    return np.ldexp(1.0, np.frexp(np.maximum(np.abs(v), 2.0 ** -126))[1] - 8)


def assert_bf16_close(got_bits, ref_bits, what: str, max_ulp: int = 1, abs_floor=None, mag=None):
    """|got - ref| <= max_ulp * (half a BF16 step of |ref| + half a step of
    |got|), i.e. one rounding on each side, each at its own binade, plus
    abs_floor (the propagated error of the GPU's fp32 sum and of differing
    inputs, where given). With `mag` (the sum of |terms| of each output),
    reports the largest error beyond the roundings and abs_floor's non-MFMA
    part as a fraction of mag: the observed accumulation error."""
    g = mx.bf16_value(got_bits)
    r = mx.bf16_value(ref_bits)
    rnd = 0.5 * max_ulp * (_bf16_ulp(r) + _bf16_ulp(g))
    tol = rnd if abs_floor is None else rnd + abs_floor
    diff = np.abs(g - r)
    bad = diff > tol
    worst = float(np.max(diff / np.maximum(tol, 1e-300))) if diff.size else 0.0
    extra = ""
    if mag is not None and diff.size:
        acc_err = np.maximum(diff - rnd - (abs_floor - MFMA_REL * mag if abs_floor is not None else 0), 0)
        extra = f", observed accumulation error / sum|terms| {float(np.max(acc_err / np.maximum(mag, 1e-300))):.2e}"
    print(f"  {what}: bits equal {float(np.mean(got_bits == ref_bits)):.4f}, beyond tol {int(bad.sum())}, "
          f"largest |diff| / tolerance {worst:.3f}{extra}", flush=True)
    if bad.any():
        idx = np.argsort((diff / np.maximum(tol, 1e-300)).ravel())[-3:]
        for i in idx:
            print(f"    got {g.ravel()[i]:.6e} ref {r.ravel()[i]:.6e} diff {diff.ravel()[i]:.3e} "
                  f"rounding {rnd.ravel()[i]:.3e} floor "
                  f"{(abs_floor.ravel()[i] if abs_floor is not None else 0):.3e}"
                  + (f" mag {mag.ravel()[i]:.3e}" if mag is not None else ""), flush=True)
    assert not bad.any(), f"{what}: {int(bad.sum())} values beyond tolerance"


def rel_l2_cos(got: np.ndarray, ref: np.ndarray):
    got = got.astype(np.float64).ravel()
    ref = ref.astype(np.float64).ravel()
    nr = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / max(nr, 1e-300)
    cos = float(got @ ref / max(np.linalg.norm(got) * nr, 1e-300))
    return rel, cos


def assert_layer_close(got_bits, ref_bits, what: str, rel_max=2e-2, cos_min=0.999):
    """The layer-output bar: rel-L2 <= 2e-2 and cosine >= 0.999."""
    g, r = mx.bf16_value(got_bits), mx.bf16_value(ref_bits)
    rel, cos = rel_l2_cos(g, r)
    eq = float(np.mean(np.asarray(got_bits) == np.asarray(ref_bits)))
    print(f"  {what}: rel-L2 {rel:.3e} cosine {cos:.7f} bits equal {eq:.4f}", flush=True)
    if np.linalg.norm(r) == 0:
        assert np.all(g == 0), what
        return
    assert rel <= rel_max and cos >= cos_min, f"{what}: rel-L2 {rel:.3e} cosine {cos:.6f}"
