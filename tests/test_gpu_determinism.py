"""Repeatability and layout checks (GPU).

* The layer gives bit-identical results when run again and again, alone and
  while other work shares the GPU (a different schedule of the same grid):
  the results must not depend on which workgroup finishes first (every
  cross-wave sum has a fixed order).
* The prepacked weight layout: every byte of the logical MX codes and scales
  lands exactly where the documented [group][unit][K-tile][tile][lane] layout
  puts it, and nowhere else.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("routed_grouped_gemm_amd")
from gpu_util import banner, dev, host  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


RUNS = [
    # decode share at T = 128 (weight-streaming GEMMs, router + grouping kernels)
    ("decode", dict(), 0),
    # a quarter of the prefill shape: LDS-tiled GEMMs with several work items
    # per workgroup and the transposed copy
    ("prefill", dict(T=4096), 1),
]


@pytest.mark.parametrize("name,kw,transpose", RUNS, ids=[r[0] for r in RUNS])
def test_layer_repeats_bit_identical(name, kw, transpose):
    """40 runs, bit-identical: 20 alone, and 20 while another stream keeps
    part of the GPU busy with large matrix products, so that the layer's
    workgroups start and finish in a different order."""
    from synth import device
    c = replace(synth.config(name, 128 if name == "decode" else None), **kw)
    banner(f"repeatability {name} T={c.T} H={c.H} I={c.I} E={c.E} k={c.k}")
    dw = device.build_weights(c)
    logits, xq, xs = device.build_inputs(c)
    flags = moe.MOE_W1_WRITE_TRANSPOSE if transpose else 0
    hT = (None, None)
    if transpose:
        ld = moe.moe_transposed_ld(c.R_max, c.G)
        hT = (torch.zeros((c.I, ld), dtype=torch.uint8, device="cuda"),
              torch.zeros((c.I, ld // 32), dtype=torch.uint8, device="cuda"))
    side = torch.cuda.Stream()
    a = torch.randn((4096, 4096), device="cuda")
    b = torch.randn((4096, 4096), device="cuda")
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I, c.shared, flags)
    first = None
    for rep in range(40):
        busy = rep >= 20
        if busy:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(6):
                    a = torch.mm(a, b) * (1.0 / 64)
        ws.buf.fill_(0xA5)                          # nothing may survive from the last run
        out = moe.moe_layer(logits, xq, xs, dw.w1, dw.w2, c.k, c.e0, c.n_local, dw.shared, flags,
                            ws=ws, hTq=hT[0], hTs=hT[1])
        got = [host(out), host(ws.view("hq")), host(ws.view("hs")), host(ws.view("y"))] + \
              ([host(hT[0]), host(hT[1])] if transpose else [])
        if first is None:
            first = got
            continue
        for i, (x, y) in enumerate(zip(first, got)):
            assert np.array_equal(x, y), f"run {rep} ({'beside other work' if busy else 'alone'}) " \
                                         f"differs from run 0 in result {i}"
    torch.cuda.synchronize()


def _expected_prepack(q, sc, fmt, is_w1):
    """The documented layout, written out with index arithmetic: group g at
    g * S; within it [unit][K-tile][tile][lane] data (FP4: 16 bytes per lane,
    K [128 kt + 32 (l/16), +32); FP8: two 16-byte halves, K [128 kt + 16 (l/16),
    +16) and +64), then [unit][K-tile/4][tile][lane][K-tile % 4] scale bytes
    (127 past the last K-tile). W1 units pair gate rows [32u, +32) (tiles 0, 1)
    with up rows I + [32u, +32) (tiles 2, 3)."""
    G, N = q.shape[0], q.shape[1]
    K = sc.shape[2] * 32
    units, kt_n = N // 64, K // 128
    kt4 = (kt_n + 3) // 4
    bpl = 16 if fmt == moe.MOE_FMT_MXFP4 else 32
    dpu = kt_n * 4 * 64 * bpl
    spu = kt4 * 4 * 64 * 4
    S = (dpu + spu) * units
    out = np.zeros(G * S, np.uint8)
    for g in range(G):
        for u in range(units):
            for t in range(4):
                for r in range(16):
                    row = (64 * u + 16 * t + r) if not is_w1 else \
                          ((N // 2 if t >= 2 else 0) + 32 * u + 16 * (t & 1) + r)
                    for kt in range(kt_n):
                        for grp in range(4):
                            lane = 16 * grp + r
                            o = g * S + u * dpu + (kt * 4 + t) * 64 * bpl + lane * 16
                            if bpl == 16:
                                out[o:o + 16] = q[g, row, kt * 64 + 16 * grp: kt * 64 + 16 * grp + 16]
                            else:
                                b = kt * 128 + 16 * grp
                                out[o:o + 16] = q[g, row, b:b + 16]
                                out[o + 1024:o + 1040] = q[g, row, b + 64:b + 80]
                    for k4 in range(kt4):
                        for grp in range(4):
                            lane = 16 * grp + r
                            o = g * S + units * dpu + u * spu + ((k4 * 4 + t) * 64 + lane) * 4
                            for j in range(4):
                                kt = 4 * k4 + j
                                out[o + j] = sc[g, row, 4 * kt + grp] if kt < kt_n else 127
    return out


@pytest.mark.parametrize("fmt,is_w1,G,N,K", [
    (0, True, 2, 128, 640),      # FP4 W1: gate/up pairing, 5 K-tiles (a partial group of 4)
    (1, False, 2, 192, 384),     # FP8 W2: three units, 3 K-tiles
    (1, True, 1, 64, 256),
])
def test_prepack_layout(fmt, is_w1, G, N, K):
    banner(f"prepack layout fmt={fmt} is_w1={is_w1} G={G} N={N} K={K}")
    rng = np.random.default_rng(N + K)
    kb = K // 2 if fmt == moe.MOE_FMT_MXFP4 else K
    q = rng.integers(0, 256, (G, N, kb), dtype=np.uint8)
    sc = rng.integers(0, 255, (G, N, K // 32), dtype=np.uint8)
    pw = moe.PackedWeights(dev(q), dev(sc), fmt, is_w1)
    got = host(pw.buf)
    want = _expected_prepack(q, sc, fmt, is_w1)
    assert got.shape == want.shape
    np.testing.assert_array_equal(got, want)
