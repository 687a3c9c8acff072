"""Exact metamorphic relations of the layer, checked on the GPU against the
GPU's own output (no oracle involved), for the decode-shaped and the
LDS-tiled GEMM kernels:

* adding 1 to every W2 scale code doubles every output exactly (the E8M0
  scale multiplies each product by a power of two, which commutes with
  every rounding in the path);
* adding 1 to the scale codes of the up half of W1 (rows [I, 2I), which
  enter SwiGLU linearly) leaves the h codes unchanged, adds 1 to the h
  scales of every nonzero block and doubles every output exactly;
* permuting the tokens (logits and x rows together) permutes the output
  rows bit for bit: each row's arithmetic does not depend on where its
  token lands in a group or a tile.

The method's definition (the GC-MoE page's layer: SwiGLU of the W1 halves,
MX block scales) fixes these relations; they pin the kernels independently
of the oracle.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import mx
import synth

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("routed_grouped_gemm_amd")
from gpu_util import banner, dev, host  # noqa: E402

FMT = {"e2m1": moe.MOE_FMT_MXFP4, "e4m3": moe.MOE_FMT_MXFP8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # a few rows per expert: the decode-shaped kernels
    ("decode-kernels", dict(T=40, H=1024, I=512, E=32, k=4, e0=8, n_local=12)),
    # about 275 rows per expert, MXFP8 weights: the LDS-tiled kernels
    ("tiled-kernels", dict(T=1100, H=512, I=384, E=8, k=2, n_local=8, w_fmt="e4m3")),
]


def _bf16_float(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _run(c, lg, xq, xs, w1, w2):
    pw1 = moe.PackedWeights(dev(np.stack([a[0] for a in w1])), dev(np.stack([a[1] for a in w1])),
                            FMT[c.w_fmt], True)
    pw2 = moe.PackedWeights(dev(np.stack([a[0] for a in w2])), dev(np.stack([a[1] for a in w2])),
                            FMT[c.w_fmt], False)
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I)
    out = moe.moe_layer(dev(lg), dev(xq), dev(xs), pw1, pw2, c.k, c.e0, c.n_local, ws=ws)
    R = int(host(ws.view("offsets"))[-1])
    return host(out).copy(), host(ws.view("hq"))[:R].copy(), host(ws.view("hs"))[:R].copy()


@pytest.mark.parametrize("name,kw", CASES, ids=[n for n, _ in CASES])
def test_layer_metamorphic_relations(name, kw):
    c = replace(synth.config("tiny"), **kw)
    banner(f"metamorphic {name} {c}")
    lg = synth.logits(c)
    xq, xs = mx.quantize_mx(synth.x(c), mx.FMT_E4M3)
    w1 = [mx.quantize_mx(synth.w1(c, g), c.w_fmt) for g in range(c.n_local)]
    w2 = [mx.quantize_mx(synth.w2(c, g), c.w_fmt) for g in range(c.n_local)]
    assert max(int(s.max()) for _, s in w1 + w2) < 254          # room for +1 below the NaN code
    out, hq, hs = _run(c, lg, xq, xs, w1, w2)
    v = _bf16_float(out)
    assert np.count_nonzero(v) > 0

    # W2 scales + 1: every output doubled
    out2, _, _ = _run(c, lg, xq, xs, w1, [(q, s + 1) for q, s in w2])
    np.testing.assert_array_equal(_bf16_float(out2), 2 * v)

    # up-half W1 scales + 1: same h codes, nonzero blocks' scales + 1, outputs doubled
    w1_up = [(q, np.concatenate([s[: c.I], s[c.I:] + 1])) for q, s in w1]
    out3, hq3, hs3 = _run(c, lg, xq, xs, w1_up, w2)
    np.testing.assert_array_equal(hq3, hq)
    nz = (hq.reshape(hq.shape[0], -1, 32) & 0x7F).any(-1)
    np.testing.assert_array_equal(hs3[nz], hs[nz] + 1)
    np.testing.assert_array_equal(_bf16_float(out3), 2 * v)

    # permuted tokens: permuted output rows, bit for bit
    p = np.random.default_rng(c.T).permutation(c.T)
    out4, _, _ = _run(c, lg[p], xq[p], xs[p], w1, w2)
    np.testing.assert_array_equal(out4, out[p])
