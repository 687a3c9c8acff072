"""Pins for the oracle's grouped GEMMs, epilogue, combine and whole layer (CPU).

* brute-force dense per-token evaluation (no grouping) must equal the grouped
  computation bit for bit;
* permutation-matrix weights give a closed form that catches transposed or
  swapped operands;
* an E = k = 1 layer is a textbook SwiGLU MLP, recomputed here with PyTorch
  float64 ops and PyTorch's own float8 rounding;
* exact metamorphic relations (power-of-two scale changes, token order);
* the transposed copy against a scalar brute-force quantiser.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe, mx
import synth


def _quantized_inputs(c, variant=0, shared=False):
    lg = synth.logits(c, variant)
    xq, xs = mx.quantize_mx(synth.x(c, variant), mx.FMT_E4M3)
    w1 = [mx.quantize_mx(synth.w1(c, g), c.w_fmt) for g in range(c.n_local)]
    w2 = [mx.quantize_mx(synth.w2(c, g), c.w_fmt) for g in range(c.n_local)]
    sh = None
    if shared:
        a = mx.quantize_mx(synth.shared_w1(c), c.w_fmt)
        b = mx.quantize_mx(synth.shared_w2(c), c.w_fmt)
        sh = (a[0], a[1], b[0], b[1])
    return (lg, xq, xs, [a[0] for a in w1], [a[1] for a in w1],
            [a[0] for a in w2], [a[1] for a in w2], sh)


def _small(name="tiny", **kw):
    from dataclasses import replace
    return replace(synth.config(name), **kw)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(T=9, E=32, k=4, e0=8, n_local=12),
    dict(T=5, E=16, k=3, e0=0, n_local=16, shared=True),
    dict(T=6, E=8, k=2, w_fmt="e4m3"),
])
def test_grouped_equals_dense(kw):
    c = _small(**kw)
    lg, xq, xs, w1q, w1s, w2q, w2s, sh = _quantized_inputs(c, shared=c.shared)
    lay = moe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I,
                        e0=c.e0, n_local=c.n_local, shared=sh)
    ref = moe.dense_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I,
                          e0=c.e0, n_local=c.n_local, shared=sh)
    np.testing.assert_array_equal(lay.out, ref)
    assert np.count_nonzero(lay.out) > 0


def _perm_matrix_fp4(perm, rows, cols):
    codes = np.zeros((rows, cols), np.uint8)
    codes[np.arange(rows), perm] = 0x2            # E2M1 1.0
    return mx.pack_fp4(codes), np.full((rows, cols // 32), 127, np.uint8)


def test_permutation_weights_closed_form():
    H = I = 256
    T = 8
    rng = np.random.default_rng(4)
    sg, su, s2 = rng.permutation(H), rng.permutation(H), rng.permutation(I)
    g_q, g_s = _perm_matrix_fp4(sg, I, H)
    u_q, u_s = _perm_matrix_fp4(su, I, H)
    w1q = [np.concatenate([g_q, u_q])]
    w1s = [np.concatenate([g_s, u_s])]
    w2q, w2s = _perm_matrix_fp4(s2, H, I)
    xq, xs = mx.quantize_mx(rng.standard_normal((T, H)), mx.FMT_E4M3)
    lg = rng.standard_normal((T, 1)).astype(np.float32)
    lay = moe.moe_layer(lg, xq, xs, 1, w1q, w1s, [w2q], [w2s], mx.FMT_E2M1, I)
    X = mx.dequantize_mx(xq, xs, mx.FMT_E4M3)
    xt = torch.from_numpy(X)
    h = (torch.nn.functional.silu(xt[:, sg]) * xt[:, su]).numpy()     # routing weight is 1
    hq, hs = mx.quantize_mx(h, mx.FMT_E4M3)
    np.testing.assert_array_equal(lay.w1.hq, hq)
    hd = mx.dequantize_mx(hq, hs, mx.FMT_E4M3)
    want = mx.bf16_rne(hd[:, s2])
    np.testing.assert_array_equal(lay.out, want)


def _torch_mx_e4m3(v):
    """MX-E4M3 quantisation written with PyTorch: shared exponent from
    torch.frexp, elements by PyTorch's float8_e4m3fn rounding."""
    t = torch.from_numpy(v).reshape(v.shape[0], -1, 32)
    amax = t.abs().amax(-1)
    _, e = torch.frexp(amax)
    E = torch.where(amax > 0, (e - 1) - 8, torch.full_like(e, -127)).clamp(-127, 127)
    scaled = t / torch.pow(2.0, E.double()).unsqueeze(-1)
    codes = scaled.clamp(-448, 448).float().to(torch.float8_e4m3fn)
    deq = codes.double() * torch.pow(2.0, E.double()).unsqueeze(-1)
    return codes.view(torch.uint8).reshape(v.shape).numpy(), (E + 127).to(torch.uint8).numpy(), \
        deq.reshape(v.shape).numpy()


def test_single_expert_is_textbook_swiglu():
    c = _small(T=12, E=1, k=1, n_local=1)
    lg, xq, xs, w1q, w1s, w2q, w2s, _ = _quantized_inputs(c)
    lay = moe.moe_layer(lg, xq, xs, 1, w1q, w1s, w2q, w2s, c.w_fmt, c.I)
    X = torch.from_numpy(mx.dequantize_mx(xq, xs, mx.FMT_E4M3))
    W1 = torch.from_numpy(mx.dequantize_mx(w1q[0], w1s[0], c.w_fmt))
    W2 = torch.from_numpy(mx.dequantize_mx(w2q[0], w2s[0], c.w_fmt))
    Wg, Wu = W1[: c.I], W1[c.I:]
    h = torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)
    hq, hs, hd = _torch_mx_e4m3(h.numpy())
    np.testing.assert_array_equal(lay.w1.hq, hq)
    np.testing.assert_array_equal(lay.w1.hs, hs)
    y = torch.from_numpy(hd) @ W2.T
    got = mx.bf16_value(lay.out)
    ulp = np.ldexp(1.0, np.frexp(np.abs(y.numpy()))[1] - 8)
    assert np.all(np.abs(got - y.numpy()) <= 0.5 * ulp + 1e-300)
    # and the unquantised SwiGLU MLP agrees to the accuracy of FP8 h
    yf = ((torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)) @ W2.T).numpy()
    cos = (got * yf).sum() / np.linalg.norm(got) / np.linalg.norm(yf)
    assert cos > 0.999


def test_metamorphic_power_of_two_scales_and_token_order():
    c = _small(T=10, E=8, k=2)
    lg, xq, xs, w1q, w1s, w2q, w2s, _ = _quantized_inputs(c)
    base = moe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I)
    v0 = mx.bf16_value(base.out)
    # W2 scales + 1 doubles every output exactly
    lay = moe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, [s + 1 for s in w2s], c.w_fmt, c.I)
    np.testing.assert_array_equal(mx.bf16_value(lay.out), 2 * v0)
    # up-half W1 scales + 1: same h codes, scales + 1, output doubled
    w1s_up = [np.concatenate([s[: c.I], s[c.I:] + 1]) for s in w1s]
    lay = moe.moe_layer(lg, xq, xs, c.k, w1q, w1s_up, w2q, w2s, c.w_fmt, c.I)
    np.testing.assert_array_equal(lay.w1.hq, base.w1.hq)
    nz = base.w1.h.reshape(base.w1.h.shape[0], -1, 32).any(-1)
    np.testing.assert_array_equal(lay.w1.hs[nz], base.w1.hs[nz] + 1)
    np.testing.assert_array_equal(mx.bf16_value(lay.out), 2 * v0)
    # permuting tokens permutes output rows
    p = np.random.default_rng(0).permutation(c.T)
    lay = moe.moe_layer(lg[p], xq[p], xs[p], c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I)
    np.testing.assert_array_equal(lay.out, base.out[p])


def test_no_local_slot_gives_zero_row():
    c = _small(T=6, E=64, k=2, e0=0, n_local=2)
    lg, xq, xs, w1q, w1s, w2q, w2s, _ = _quantized_inputs(c)
    lay = moe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I, e0=0, n_local=2)
    none = (lay.perm.slot_row < 0).all(1)
    assert none.any()
    assert np.all(lay.out[none] == 0)


def test_transposed_copy_against_scalar_quantiser():
    c = _small(T=30, E=2, k=2, transpose=True)       # both experts get 30 rows
    lg, xq, xs, w1q, w1s, w2q, w2s, _ = _quantized_inputs(c)
    c2 = _small(T=45, E=2, k=1)
    lg2 = synth.logits(c2)
    xq2, xs2 = mx.quantize_mx(synth.x(c2), mx.FMT_E4M3)
    for L, XQ, XS, k in [(lg, xq, xs, 2), (lg2, xq2, xs2, 1)]:
        lay = moe.moe_layer(L, XQ, XS, k, w1q, w1s, w2q, w2s, c.w_fmt, c.I, transpose=True)
        for g in range(2):
            lo, hi = lay.perm.offsets[g], lay.perm.offsets[g + 1]
            h = lay.w1.h[lo:hi]
            n = hi - lo
            n32 = -(-n // 32) * 32
            q, s = lay.w1.hTq[g], lay.w1.hTs[g]
            assert q.shape == (c.I, n32) and s.shape == (c.I, n32 // 32)
            assert np.all(q[:, n:] == 0)
            for f in range(0, c.I, 37):
                for b in range(n32 // 32):
                    vals = list(h[b * 32: min(n, b * 32 + 32), f])
                    amax = max(abs(v) for v in vals)
                    E = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
                    assert s[f, b] == E + 127
                    for i, v in enumerate(vals):
                        want = mx.encode(np.array(v / 2.0 ** E), mx.FMT_E4M3)
                        assert q[f, b * 32 + i] == want


def test_weight_at_combine_variant_close():
    c = _small(T=8, E=8, k=2)
    lg, xq, xs, w1q, w1s, w2q, w2s, _ = _quantized_inputs(c)
    a = mx.bf16_value(moe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I).out)
    b = mx.bf16_value(moe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I,
                                    weight_at_combine=True).out)
    # Both placements compute sum_j w_j E_j(x); they differ only in where the
    # FP8 rounding of h happens (relative error <= 2^-4 per element each).
    assert np.linalg.norm(a - b) / np.linalg.norm(a) < 2.0 ** -3


@pytest.mark.parametrize("kw", [dict(T=8, E=8, k=2), dict(T=7, E=16, k=3, e0=4, n_local=8, shared=True)])
def test_weight_at_combine_equals_dense(kw):
    """The weight-at-combine placement, grouped, equals the per-token brute
    force that applies each routing weight to the expert's BF16 output: bit
    for bit."""
    c = _small(**kw)
    lg, xq, xs, w1q, w1s, w2q, w2s, sh = _quantized_inputs(c, shared=c.shared)
    lay = moe.moe_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I, e0=c.e0,
                        n_local=c.n_local, shared=sh, weight_at_combine=True)
    ref = moe.dense_layer(lg, xq, xs, c.k, w1q, w1s, w2q, w2s, c.w_fmt, c.I, e0=c.e0,
                          n_local=c.n_local, shared=sh, weight_at_combine=True)
    np.testing.assert_array_equal(lay.out, ref)
    # and the unweighted h: every routed row's h equals the shared-weight-1 MLP
    r = int(lay.perm.offsets[1])
    if r:
        x0 = mx.dequantize_mx(xq[lay.perm.row_src[:1]], xs[lay.perm.row_src[:1]], mx.FMT_E4M3)
        acc = x0 @ mx.dequantize_mx(w1q[0], w1s[0], c.w_fmt).T
        np.testing.assert_array_equal(lay.w1.h[:1], moe.swiglu_rows(acc, c.I, np.ones(1)))


def test_algorithmic_work_formulas():
    # decode share, T=1, one active expert: 4*256 logits + 7168*(1+1/32) x +
    # 3*2048*7168*(0.5 + 1/32) weights + 2*7168 out
    b = moe.algorithmic_bytes(1, 256, 7168, 2048, 1, mx.FMT_E2M1)
    assert b == 1024 + 7168 + 224 + (3 * 2048 * 7168 // 2 + 3 * 2048 * 224) + 14336
    assert moe.algorithmic_flops(10, 7168, 2048) == 6 * 10 * 7168 * 2048
