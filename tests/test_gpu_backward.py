"""Epilogue variants of the fused W1 epilogue and its backward against the
oracle (GPU).

* grouped W1 with GeGLU, squared ReLU, Swish with slope beta, bias and clamp
  (both kernel families), and the BF16 copy of the pre-activation;
* a whole layer with a variant;
* the backward GEMM + dActivation + MX quantisation (rows and 32-row
  transposed blocks) + routing-weight gradient, for each activation, with
  and without the clamp, FP8 and FP4 transposed W2, including a partial last
  256-wide weight tile (I not a multiple of 256) and several work items per
  workgroup.
"""
import numpy as np
import pytest
import torch

from oracle import moe as omoe, mx
import synth

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("routed_grouped_gemm_amd")
from gpu_util import (MFMA_REL, assert_bf16_close, assert_layer_close, assert_mx_within_1ulp,  # noqa: E402
                      banner, bf16_bits, dev, host)

FMT = {"e2m1": moe.MOE_FMT_MXFP4, "e4m3": moe.MOE_FMT_MXFP8}
# relative error of the GPU's fp32 activation functions (exp, erf, division)
ACT_REL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _packed(ws, fmt, is_w1):
    return moe.PackedWeights(dev(np.stack([a[0] for a in ws])), dev(np.stack([a[1] for a in ws])),
                             FMT[fmt], is_w1)


def _act_bound(g, u, dg, du, act, beta):
    """|a(g') u' - a(g) u| for |g' - g| <= dg, |u' - u| <= du: the derivative
    bound over the interval, plus the product term."""
    gmax = np.abs(g) + dg
    if act == omoe.ACT_SRELU:
        slope = 2 * gmax
    elif act == omoe.ACT_GEGLU:
        slope = np.full_like(g, 1.13)
    else:
        slope = np.full_like(g, 1.1 * max(beta, 1.0))
    amax = np.abs(omoe.activation(g, act, beta)) + slope * dg
    return slope * dg * (np.abs(u) + du) + amax * du


VARIANTS = [
    ("geglu", dict(act=omoe.ACT_GEGLU)),
    ("srelu-clamp", dict(act=omoe.ACT_SRELU, limit=0.75)),
    ("swish-beta-clamp", dict(act=omoe.ACT_SWIGLU, beta=1.702, limit=1.5)),
]


@pytest.mark.parametrize("kernel", ["streamed", "pass", "tiled"])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("name,var", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_w1_variant_parity(name, var, bias, kernel):
    banner(f"W1 variant {name} bias={bias} {kernel}")
    rng = np.random.default_rng(17)
    counts = [40, 0, 300, 17, 5]
    H, I, fmt = 512, 256, "e4m3" if kernel == "tiled" else "e2m1"
    G = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    c = synth.Config("stage", 1, H, I, G, 1, 0, G, fmt, "normal", seed=31)
    xq, xs = mx.quantize_mx(rng.standard_normal((R, H)), mx.FMT_E4M3)
    row_w = rng.uniform(0.1, 1.0, R).astype(np.float32)
    w1 = [mx.quantize_mx(synth.w1(c, g), fmt) for g in range(G)]
    b = (rng.standard_normal((G, 2 * I)) * 0.5).astype(np.float32) if bias else None
    epi = dict(var, bias=None if b is None else b.astype(np.float64))
    ref = omoe.grouped_w1(xq, xs, offsets, row_w.astype(np.float64), [a[0] for a in w1],
                          [a[1] for a in w1], fmt, I, **epi)
    pre = torch.zeros((R, 2 * I), dtype=torch.int16, device="cuda").view(torch.uint16)
    e = moe.Epilogue(act=var["act"], beta=var.get("beta", 1.0), limit=var.get("limit", 0.0),
                     bias=None if b is None else dev(b), save_pre=pre)
    flags = {"streamed": moe.MOE_GEMM_STREAMED, "pass": moe.MOE_GEMM_PASS, "tiled": moe.MOE_GEMM_TILED}[kernel]
    hq, hs, _, _ = moe.moe_grouped_w1(_packed(w1, fmt, True), dev(np.array(counts, np.int32)), dev(offsets),
                                      dev(row_w), dev(xq), dev(xs), I, flags, epi=e)
    # error bound of the fp32 sums, through bias, clamp and the activation
    X = np.abs(mx.dequantize_mx(xq, xs, mx.FMT_E4M3))
    mag = np.zeros((R, 2 * I))
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            mag[lo:hi] = X[lo:hi] @ np.abs(mx.dequantize_mx(w1[g][0], w1[g][1], fmt)).T
    gz, uz = omoe.preactivation(ref.acc, I, None, 0.0)
    if b is not None:
        for g in range(G):
            lo, hi = offsets[g], offsets[g + 1]
            gz[lo:hi] += b[g, :I]
            uz[lo:hi] += b[g, I:]
    lim = var.get("limit", 0.0)
    gc = np.clip(gz, -lim, lim) if lim else gz
    uc = np.clip(uz, -lim, lim) if lim else uz
    dh = _act_bound(gc, uc, MFMA_REL * mag[:, :I] + 1e-6 * np.abs(gz), MFMA_REL * mag[:, I:] + 1e-6 * np.abs(uz),
                    var["act"], var.get("beta", 1.0)) * row_w[:, None] + (ACT_REL + 2e-5) * np.abs(ref.h)
    assert_mx_within_1ulp(host(hq)[:R], host(hs)[:R], ref.hq, ref.hs, f"h ({name})", extra_tol=dh)
    # the saved pre-activation: BF16 of the GEMM output plus the bias
    pre_ref = mx.bf16_rne(np.concatenate([gz, uz], axis=1))
    assert_bf16_close(bf16_bits(pre)[:R], pre_ref, "pre-activation", abs_floor=MFMA_REL * mag)


def test_layer_with_variant():
    from dataclasses import replace
    c = replace(synth.config("tiny"), T=40, E=8, k=2, shared=True)
    banner(f"layer variant {c}")
    lg = synth.logits(c)
    xq, xs = mx.quantize_mx(synth.x(c), mx.FMT_E4M3)
    w1 = [mx.quantize_mx(synth.w1(c, g), c.w_fmt) for g in range(c.n_local)]
    w2 = [mx.quantize_mx(synth.w2(c, g), c.w_fmt) for g in range(c.n_local)]
    a, bb = mx.quantize_mx(synth.shared_w1(c), c.w_fmt), mx.quantize_mx(synth.shared_w2(c), c.w_fmt)
    b = (np.random.default_rng(4).standard_normal((c.G, 2 * c.I)) * 0.3).astype(np.float32)
    epi = dict(act=omoe.ACT_GEGLU, limit=2.0, bias=b.astype(np.float64))
    ref = omoe.moe_layer(lg, xq, xs, c.k, [q for q, _ in w1], [s for _, s in w1], [q for q, _ in w2],
                         [s for _, s in w2], c.w_fmt, c.I, n_local=c.n_local,
                         shared=(a[0], a[1], bb[0], bb[1]), epi=epi)
    shared = (moe.PackedWeights(dev(a[0][None]), dev(a[1][None]), FMT[c.w_fmt], True),
              moe.PackedWeights(dev(bb[0][None]), dev(bb[1][None]), FMT[c.w_fmt], False))
    e = moe.Epilogue(act=moe.MOE_ACT_GEGLU, limit=2.0, bias=dev(b))
    out = moe.moe_layer(dev(lg), dev(xq), dev(xs), _packed(w1, c.w_fmt, True), _packed(w2, c.w_fmt, False),
                        c.k, c.e0, c.n_local, shared, epi=e)
    assert_layer_close(bf16_bits(out), ref.out, "out (GeGLU, clamp, bias)")


BWD = [
    # counts, H, I, W2T format, act, beta, limit, flags
    ([40, 0, 300, 17, 260], 512, 256, "e4m3", omoe.ACT_SWIGLU, 1.0, 0.0, "transpose"),
    ([40, 0, 300, 17, 260], 512, 384, "e2m1", omoe.ACT_GEGLU, 1.0, 0.0, "transpose"),     # partial tile
    ([129, 3, 700], 768, 256, "e4m3", omoe.ACT_SRELU, 1.0, 1.25, "transpose,no-weight"),
    ([5, 64, 33], 512, 256, "e4m3", omoe.ACT_SWIGLU, 1.702, 2.0, ""),
    # about 290 work items over 256 workgroups: some take two; 22 units = 5.5 tiles
    ([5000, 257, 0, 3100, 2555, 1031], 256, 1408, "e4m3", omoe.ACT_SWIGLU, 1.0, 0.0, "transpose"),
]


@pytest.mark.parametrize("counts,H,I,fmt,act,beta,limit,opts", BWD)
def test_backward_parity(counts, H, I, fmt, act, beta, limit, opts):
    banner(f"backward counts={counts} H={H} I={I} {fmt} act={act} beta={beta} limit={limit} {opts}")
    rng = np.random.default_rng(sum(counts) + I)
    G = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    T = max(R // 3, 1)
    transpose = "transpose" in opts
    weighted = "no-weight" not in opts
    dyq, dys = mx.quantize_mx(rng.standard_normal((T, H)), mx.FMT_E4M3)
    row_src = rng.integers(0, T, R).astype(np.int32)
    w2t = [mx.quantize_mx(rng.standard_normal((I, H)) * 0.05, fmt) for _ in range(G)]
    pre_bits = mx.bf16_rne(rng.standard_normal((R, 2 * I)) * 1.5)
    row_w = rng.uniform(0.1, 1.0, R).astype(np.float32)
    ref = omoe.grouped_w1_backward(dyq, dys, row_src, offsets, row_w.astype(np.float64) if weighted else np.ones(R),
                                   pre_bits, [q for q, _ in w2t], [s for _, s in w2t], fmt, I, act, beta, limit,
                                   transpose=transpose)
    e = moe.Epilogue(act=act, beta=beta, limit=limit)
    off32 = np.concatenate([[0], np.cumsum((np.array(counts) + 31) // 32 * 32)]).astype(np.int32)
    res = moe.moe_grouped_w1_backward(_packed(w2t, fmt, False), dev(np.array(counts, np.int32)), dev(offsets),
                                      dev(row_w) if weighted else None, dev(dyq), dev(dys), dev(row_src),
                                      dev(pre_bits.view(np.int16)).view(torch.uint16), I, epi=e,
                                      flags=moe.MOE_W1_WRITE_TRANSPOSE if transpose else 0,
                                      offsets32=dev(off32), want_dw=weighted)
    # error of the GPU's dh (fp32 sum) through the derivative
    D = np.abs(mx.dequantize_mx(dyq, dys, mx.FMT_E4M3))
    mag = np.zeros((R, I))
    for g in range(G):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            mag[lo:hi] = D[row_src[lo:hi]] @ np.abs(mx.dequantize_mx(w2t[g][0], w2t[g][1], fmt)).T
    ddh = MFMA_REL * mag
    pre = mx.bf16_value(pre_bits)
    g_, u_ = pre[:, :I], pre[:, I:]
    gc = np.clip(g_, -limit, limit) if limit else g_
    uc = np.clip(u_, -limit, limit) if limit else u_
    w = row_w[:, None] if weighted else 1.0
    tol_g = ddh * np.abs(uc * omoe.activation_grad(gc, act, beta)) * w
    tol_u = ddh * np.abs(omoe.activation(gc, act, beta)) * w
    tol = np.concatenate([tol_g, tol_u], axis=1) + (ACT_REL + 1e-6) * np.abs(ref.d)
    assert_mx_within_1ulp(host(res["dq"])[:R], host(res["ds"])[:R], ref.dq, ref.ds, "d rows", extra_tol=tol)
    if transpose:
        q_ref, s_ref = omoe.concat_transposed(ref.dTq, ref.dTs, 2 * I)
        n = q_ref.shape[1]
        tT = np.zeros((2 * I, n))
        col = 0
        for g in range(G):
            lo, hi = offsets[g], offsets[g + 1]
            tT[:, col:col + hi - lo] = tol[lo:hi].T
            col += (hi - lo + 31) // 32 * 32
        assert_mx_within_1ulp(host(res["dTq"])[:, :n], host(res["dTs"])[:, :n // 32], q_ref, s_ref, "d transposed",
                              extra_tol=tT)
    if weighted:
        got = host(res["dw"])[:R].astype(np.float64)
        au = np.abs(omoe.activation(gc, act, beta) * uc)
        bound = np.sum(ddh * au, axis=1) + (ACT_REL + 1e-6) * np.sum(np.abs(ref.dh) * au, axis=1)
        err = np.abs(got - ref.dw)
        print(f"  dw: largest |diff| / bound {float(np.max(err / np.maximum(bound, 1e-300))):.3f}", flush=True)
        assert np.all(err <= bound), f"dw: {int(np.sum(err > bound))} beyond the bound"
