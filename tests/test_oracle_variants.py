"""Pins for the oracle's epilogue variants and the backward of the fused W1
epilogue (CPU).

* the activations at printed values of the normal distribution and other
  closed forms, and against PyTorch's own float64 GELU / SiLU / ReLU;
* their derivatives against central finite differences;
* the backward rows (dg, du, dw) against PyTorch autograd of the forward,
  written independently with torch ops, with bias and clamp;
* the backward GEMM against a loop brute force on tiny inputs;
* grouped forward with each variant equals the per-token dense evaluation.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe, mx
import synth

ACTS = [moe.ACT_SWIGLU, moe.ACT_GEGLU, moe.ACT_SRELU]


def test_activation_closed_forms():
    # the standard normal CDF at 1 and 1.96 (printed in every normal table)
    assert abs(moe.activation(1.0, moe.ACT_GEGLU) - 0.8413447460685429) < 1e-15
    assert abs(moe.activation(1.959963984540054, moe.ACT_GEGLU) / 1.959963984540054 - 0.975) < 1e-12
    assert moe.activation(0.0, moe.ACT_GEGLU) == 0.0
    assert abs(moe.activation(-1.0, moe.ACT_GEGLU) + (1 - 0.8413447460685429)) < 1e-15
    # Swish_beta(1) = 1 / (1 + e^-beta)
    for beta in (1.0, 2.0, 0.5):
        assert abs(moe.activation(1.0, moe.ACT_SWIGLU, beta) - 1 / (1 + math.exp(-beta))) < 1e-15
    assert moe.activation(0.0, moe.ACT_SWIGLU) == 0.0
    np.testing.assert_array_equal(moe.activation(np.array([-2.0, 0.0, 3.0]), moe.ACT_SRELU), [0.0, 0.0, 9.0])


def test_activations_against_torch():
    z = np.linspace(-9, 9, 2001)
    t = torch.from_numpy(z)
    np.testing.assert_allclose(moe.activation(z, moe.ACT_GEGLU),
                               torch.nn.functional.gelu(t, approximate="none").numpy(), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(moe.activation(z, moe.ACT_SWIGLU), torch.nn.functional.silu(t).numpy(),
                               rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(moe.activation(z, moe.ACT_SRELU), (torch.relu(t) ** 2).numpy(), rtol=0, atol=0)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("beta", [1.0, 1.7])
def test_activation_grad_finite_difference(act, beta):
    z = np.linspace(-6, 6, 997)
    z = z[np.abs(z) > 1e-3]                       # away from sReLU's kink
    eps = 1e-6
    fd = (moe.activation(z + eps, act, beta) - moe.activation(z - eps, act, beta)) / (2 * eps)
    np.testing.assert_allclose(moe.activation_grad(z, act, beta), fd, rtol=1e-7, atol=1e-8)


def _torch_forward(pre, w, I, act, beta, limit):
    g, u = pre[:, :I], pre[:, I:]
    if limit > 0:
        g, u = torch.clamp(g, -limit, limit), torch.clamp(u, -limit, limit)
    if act == moe.ACT_SWIGLU:
        a = g * torch.sigmoid(beta * g)
    elif act == moe.ACT_GEGLU:
        a = torch.nn.functional.gelu(g, approximate="none")
    else:
        a = torch.relu(g) ** 2
    return a * u * w[:, None]


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("beta,limit", [(1.0, 0.0), (1.5, 2.5)])
def test_backward_rows_against_autograd(act, beta, limit):
    rng = np.random.default_rng(7 + act)
    n, I = 12, 40
    pre = rng.standard_normal((n, 2 * I)) * 2
    pre[np.abs(np.abs(pre) - limit) < 1e-3] += 0.01     # no value on a clamp edge
    pre[np.abs(pre) < 1e-3] += 0.01                      # nor on the ReLU kink
    dh = rng.standard_normal((n, I))
    w = rng.uniform(0.1, 1.0, n)
    tp = torch.from_numpy(pre).requires_grad_(True)
    tw = torch.from_numpy(w).requires_grad_(True)
    h = _torch_forward(tp, tw, I, act, beta, limit)
    (h * torch.from_numpy(dh)).sum().backward()
    d, dw = moe.glu_backward_rows(pre, dh, I, w, act, beta, limit)
    np.testing.assert_allclose(d, tp.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dw * 1.0, tw.grad.numpy(), rtol=1e-12, atol=1e-14)
    if limit > 0:
        assert np.any(d[:, :I][np.abs(pre[:, :I]) > limit] == 0)   # clamped entries pass no gradient


def test_glu_rows_default_is_swiglu():
    rng = np.random.default_rng(3)
    acc = rng.standard_normal((5, 64))
    w = rng.uniform(0, 1, 5)
    np.testing.assert_array_equal(moe.glu_rows(acc, 32, w), moe.swiglu_rows(acc, 32, w))
    # bias is added before the clamp, to both chunks
    b = rng.standard_normal(64)
    np.testing.assert_allclose(moe.glu_rows(acc, 32, w, bias=b, limit=0.7),
                               moe.swiglu_rows(np.clip(acc + b, -0.7, 0.7), 32, w), rtol=1e-15)


@pytest.mark.parametrize("w_fmt", ["e2m1", "e4m3"])
def test_backward_gemm_brute_force(w_fmt):
    """dh by an explicit triple loop over (row, feature, K), the rest of the
    stage from it; the transposed copy per group."""
    rng = np.random.default_rng(11)
    T, H, I = 6, 64, 32
    counts = [3, 0, 5]
    G = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    row_src = rng.integers(0, T, R).astype(np.int32)
    dq, ds = mx.quantize_mx(rng.standard_normal((T, H)), mx.FMT_E4M3)
    w2t = [mx.quantize_mx(rng.standard_normal((I, H)) * 0.05, w_fmt) for _ in range(G)]
    pre_bits = mx.bf16_rne(rng.standard_normal((R, 2 * I)))
    row_w = rng.uniform(0.1, 1, R)
    out = moe.grouped_w1_backward(dq, ds, row_src, offsets, row_w, pre_bits, [a[0] for a in w2t],
                                  [a[1] for a in w2t], w_fmt, I, transpose=True)
    dd = mx.dequantize_mx(dq, ds, mx.FMT_E4M3)
    for g in range(G):
        W = mx.dequantize_mx(w2t[g][0], w2t[g][1], w_fmt)
        for r in range(offsets[g], offsets[g + 1]):
            for i in range(I):
                acc = 0.0
                for h in range(H):
                    acc += dd[row_src[r], h] * W[i, h]
                assert abs(out.dh[r, i] - acc) <= 1e-12 * max(1.0, abs(acc))
    d, dw = moe.glu_backward_rows(mx.bf16_value(pre_bits), out.dh, I, row_w)
    np.testing.assert_array_equal(out.d, d)
    np.testing.assert_array_equal(out.dw, dw)
    q, s = mx.quantize_mx(d, mx.FMT_E4M3)
    np.testing.assert_array_equal(out.dq, q)
    np.testing.assert_array_equal(out.ds, s)
    assert [x.shape for x in out.dTq] == [(2 * I, 32), (2 * I, 0), (2 * I, 32)]
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        tq, ts = moe.quantize_transposed(d[lo:hi])
        np.testing.assert_array_equal(out.dTq[g], tq)
        np.testing.assert_array_equal(out.dTs[g], ts)


VARIANTS = [
    dict(act=moe.ACT_GEGLU),
    dict(act=moe.ACT_SRELU, limit=1.5),
    dict(act=moe.ACT_SWIGLU, beta=1.702, limit=3.0),
]


@pytest.mark.parametrize("epi", VARIANTS)
@pytest.mark.parametrize("with_bias", [False, True])
def test_variant_grouped_equals_dense(epi, with_bias):
    from dataclasses import replace
    c = replace(synth.config("tiny"), T=7, E=8, k=2, shared=True)
    lg = synth.logits(c)
    xq, xs = mx.quantize_mx(synth.x(c), mx.FMT_E4M3)
    w1 = [mx.quantize_mx(synth.w1(c, g), c.w_fmt) for g in range(c.n_local)]
    w2 = [mx.quantize_mx(synth.w2(c, g), c.w_fmt) for g in range(c.n_local)]
    a, b = mx.quantize_mx(synth.shared_w1(c), c.w_fmt), mx.quantize_mx(synth.shared_w2(c), c.w_fmt)
    sh = (a[0], a[1], b[0], b[1])
    e = dict(epi)
    if with_bias:
        e["bias"] = np.random.default_rng(5).standard_normal((c.G, 2 * c.I)) * 0.3
    args = (lg, xq, xs, c.k, [q for q, _ in w1], [s for _, s in w1], [q for q, _ in w2], [s for _, s in w2],
            c.w_fmt, c.I)
    lay = moe.moe_layer(*args, n_local=c.n_local, shared=sh, epi=e)
    ref = moe.dense_layer(*args, n_local=c.n_local, shared=sh, epi=e)
    np.testing.assert_array_equal(lay.out, ref)
    base = moe.moe_layer(*args, n_local=c.n_local, shared=sh)
    assert not np.array_equal(lay.out, base.out)          # the variant changes the result
