"""The single-launch decode layer (at most 8 tokens) against the oracle
(GPU), and its control block: every element of h and of the output at small
shapes, with a shared expert, the weight at the combine, renormalised routing
and an epilogue variant; repeated calls on one workspace (the counters reset
at the end of every launch, the error word stays zero); a workspace full of
garbage (the block is initialised in the launch); no local rows (a zero
output); and the same results while another stream keeps the GPU busy (the
item order never needs a workgroup that is not running)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import moe as omoe, mx
import synth

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="the single-launch decode layer is switched off: its first launch ran for "
                            "minutes on the GPU, twice (the second time with wall-clock-bounded waits), "
                            "and the cause is not established; moe_layer takes the separate kernels"),
]

moe = pytest.importorskip("routed_grouped_gemm_amd")
from gpu_util import (MFMA_REL, assert_layer_close, assert_mx_within_1ulp, banner, bf16_bits,  # noqa: E402
                      dev, host)

FMT = {"e2m1": moe.MOE_FMT_MXFP4, "e4m3": moe.MOE_FMT_MXFP8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(c, flags=0, epi=None):
    lg = synth.logits(c)
    xq, xs = mx.quantize_mx(synth.x(c), mx.FMT_E4M3)
    w1 = [mx.quantize_mx(synth.w1(c, g), c.w_fmt) for g in range(c.n_local)]
    w2 = [mx.quantize_mx(synth.w2(c, g), c.w_fmt) for g in range(c.n_local)]
    sh = None
    if c.shared:
        a, b = mx.quantize_mx(synth.shared_w1(c), c.w_fmt), mx.quantize_mx(synth.shared_w2(c), c.w_fmt)
        sh = (a[0], a[1], b[0], b[1])
    ref = omoe.moe_layer(lg, xq, xs, c.k, [q for q, _ in w1], [s for _, s in w1], [q for q, _ in w2],
                         [s for _, s in w2], c.w_fmt, c.I, e0=c.e0, n_local=c.n_local, shared=sh,
                         renorm=bool(flags & moe.MOE_ROUTE_RENORM),
                         weight_at_combine=bool(flags & moe.MOE_WEIGHT_AT_COMBINE), epi=epi)
    pk = lambda ws, is_w1: moe.PackedWeights(dev(np.stack([a[0] for a in ws])),  # noqa: E731
                                             dev(np.stack([a[1] for a in ws])), FMT[c.w_fmt], is_w1)
    shared = None
    if sh is not None:
        shared = (moe.PackedWeights(dev(sh[0][None]), dev(sh[1][None]), FMT[c.w_fmt], True),
                  moe.PackedWeights(dev(sh[2][None]), dev(sh[3][None]), FMT[c.w_fmt], False))
    return (dev(lg), dev(xq), dev(xs), pk(w1, True), pk(w2, False), shared), ref, (xq, xs, w1, sh)


def _h_bound(c, ref, xq, xs, w1, sh, wts):
    X = np.abs(mx.dequantize_mx(*omoe.gather_rows(xq, xs, ref.perm), mx.FMT_E4M3))
    ws1 = list(w1) + ([(sh[0], sh[1])] if sh else [])
    mag = np.zeros_like(ref.w1.acc)
    for g in range(c.G):
        lo, hi = ref.perm.offsets[g], ref.perm.offsets[g + 1]
        if hi > lo:
            mag[lo:hi] = X[lo:hi] @ np.abs(mx.dequantize_mx(ws1[g][0], ws1[g][1], c.w_fmt)).T
    gate, up = ref.w1.acc[:, :c.I], ref.w1.acc[:, c.I:]
    dg, du = MFMA_REL * mag[:, :c.I], MFMA_REL * mag[:, c.I:]
    return (1.1 * (np.abs(up) + du) * dg + np.abs(omoe.silu(gate)) * du) * np.abs(wts)[:, None] \
        + 2e-5 * np.abs(ref.w1.h)


BASE = dict(H=1024, I=512, E=64, k=8, e0=8, n_local=16)
CASES = [
    ("one-token", dict(T=1), 0),
    ("three-shared-wc", dict(T=3, shared=True), moe.MOE_WEIGHT_AT_COMBINE),
    ("eight-renorm", dict(T=8), moe.MOE_ROUTE_RENORM),
    ("eight-ceil-fp8", dict(T=8, w_fmt="e4m3", shared=True), moe.MOE_SCALE_RULE_CEIL),
]


@pytest.mark.parametrize("name,kw,flags", CASES, ids=[c[0] for c in CASES])
def test_fused_layer_parity(name, kw, flags):
    c = replace(synth.config("tiny"), **{**BASE, **kw})
    banner(f"single-launch layer {name} {c}")
    args, ref, (xq, xs, w1, sh) = _case(c, flags)
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I, c.shared, flags)
    out = moe.moe_layer(*args[:5], c.k, c.e0, c.n_local, args[5], flags, ws=ws)
    ctrl = host(ws.view("ctrl"))
    print(f"  control block {ctrl[:8].tolist()} done/arrivals {ctrl[8:].tolist()}", flush=True)
    assert ctrl[2] == 0, f"a wait between workgroups timed out: {ctrl[:8].tolist()}"
    R = int(ref.perm.offsets[-1])
    np.testing.assert_array_equal(host(ws.view("topk_idx")), ref.topk_idx)
    np.testing.assert_array_equal(host(ws.view("counts")), ref.perm.counts)
    np.testing.assert_array_equal(host(ws.view("offsets")), ref.perm.offsets)
    np.testing.assert_array_equal(host(ws.view("slot_row")), ref.perm.slot_row)
    np.testing.assert_array_equal(host(ws.view("row_src"))[:R], ref.perm.row_src)
    wts = np.ones(R) if flags & moe.MOE_WEIGHT_AT_COMBINE else ref.perm.row_w
    if R:
        assert_mx_within_1ulp(host(ws.view("hq"))[:R], host(ws.view("hs"))[:R], ref.w1.hq, ref.w1.hs, "h",
                              extra_tol=_h_bound(c, ref, xq, xs, w1, sh, wts))
    assert_layer_close(bf16_bits(out), ref.out, "out")
    assert ctrl[3] == 0 and ctrl[4] == 0 and not ctrl[8:].any(), ctrl[:16]
    # the separate-kernel path on the same inputs agrees to the same bar
    out2 = moe.moe_layer(*args[:5], c.k, c.e0, c.n_local, args[5], flags | moe.MOE_LAYER_SEPARATE_KERNELS)
    assert_layer_close(bf16_bits(out2), ref.out, "out (separate kernels)")


def test_fused_layer_variant():
    c = replace(synth.config("tiny"), **{**BASE, "T": 6, "shared": True})
    b = (np.random.default_rng(8).standard_normal((c.G, 2 * c.I)) * 0.3).astype(np.float32)
    epi = dict(act=omoe.ACT_SRELU, limit=1.0, bias=b.astype(np.float64))
    banner(f"single-launch layer with sReLU, clamp, bias {c}")
    args, ref, _ = _case(c, 0, epi)
    e = moe.Epilogue(act=moe.MOE_ACT_SRELU, limit=1.0, bias=dev(b))
    out = moe.moe_layer(*args[:5], c.k, c.e0, c.n_local, args[5], 0, epi=e)
    assert_layer_close(bf16_bits(out), ref.out, "out (sReLU, clamp, bias)")


def test_fused_layer_no_local_rows():
    c = replace(synth.config("tiny"), **{**BASE, "T": 2, "k": 2, "n_local": 4})
    picked = set(omoe.route(synth.logits(c), c.k)[0].ravel().tolist())
    e0 = next(e for e in range(0, c.E - c.n_local + 1) if not picked & set(range(e, e + c.n_local)))
    c = replace(c, e0=e0)
    banner(f"single-launch layer without local rows {c}")
    args, ref, _ = _case(c)
    out = torch.full((c.T, c.H), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.uint16)
    moe.moe_layer(*args[:5], c.k, c.e0, c.n_local, None, 0, out=out)
    np.testing.assert_array_equal(host(out), np.zeros((c.T, c.H), np.uint16))


def test_fused_layer_repeats_and_initialises():
    """Calls 0-9 on a workspace full of garbage before each call (the block is
    initialised inside the launch), calls 10-29 on the same workspace as left
    by the previous call, 30-39 beside matrix products on another stream:
    bit-identical, error word zero, counters back at zero."""
    from synth import device
    c = synth.config("decode", 8)
    banner(f"single-launch repeats decode T={c.T}")
    dw = device.build_weights(c)
    logits, xq, xs = device.build_inputs(c)
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I)
    side = torch.cuda.Stream()
    a = torch.randn((4096, 4096), device="cuda")
    b = torch.randn((4096, 4096), device="cuda")
    first = None
    for rep in range(40):
        if rep < 10:
            ws.buf.fill_(0xA5)
        if rep >= 30:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(6):
                    a = torch.mm(a, b) * (1.0 / 64)
        out = moe.moe_layer(logits, xq, xs, dw.w1, dw.w2, c.k, c.e0, c.n_local, ws=ws)
        got = (host(out), host(ws.view("hq")), host(ws.view("y")))
        ctrl = host(ws.view("ctrl"))
        assert ctrl[2] == 0, f"run {rep}: a wait between workgroups timed out"
        assert ctrl[3] == 0 and ctrl[4] == 0 and not ctrl[8:].any(), f"run {rep}: counters not reset"
        R = int(host(ws.view("offsets"))[-1])
        got = (got[0], got[1][:R], got[2][:R])
        if first is None:
            first = got
        else:
            for i in range(3):
                assert np.array_equal(first[i], got[i]), f"run {rep} differs from run 0 in result {i}"
    torch.cuda.synchronize()
