"""The layer needs no host synchronisation and allocates nothing: it can be
captured once into a HIP graph and replayed with new inputs written into the
captured buffers (fusion blog, "Removing host-device synchronisation":
device-resident group sizes allow whole-iteration graphs; GC-MoE page,
"Developer view": the layer is replayed as a captured graph).

Each replay, with eager work and synchronisations between replays, must equal
an eager call on the same inputs bit for bit (same kernels, deterministic).
"""
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


def _packed(c, which):
    gen = synth.w1 if which == 1 else synth.w2
    ws = [mx.quantize_mx(gen(c, g), c.w_fmt) for g in range(c.n_local)]
    return moe.PackedWeights(dev(np.stack([a[0] for a in ws])), dev(np.stack([a[1] for a in ws])),
                             FMT[c.w_fmt], which == 1)


@pytest.mark.parametrize("T", [16, 100])     # fused router+grouping, and separate launches
def test_graph_replays_equal_eager(T):
    from dataclasses import replace
    c = replace(synth.config("tiny"), T=T, E=16, k=4, n_local=12, e0=2, H=512, I=256)
    banner(f"graph replay T={T}")
    w1, w2 = _packed(c, 1), _packed(c, 2)
    lg_buf = torch.empty((c.T, c.E), dtype=torch.float32, device="cuda")
    xq_buf = torch.empty((c.T, c.H), dtype=torch.uint8, device="cuda")
    xs_buf = torch.empty((c.T, c.H // 32), dtype=torch.uint8, device="cuda")
    out_buf = torch.empty((c.T, c.H), dtype=torch.uint16, device="cuda")
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer(lg_buf, xq_buf, xs_buf, w1, w2, c.k, c.e0, c.n_local, out=out_buf, ws=ws)
    ws_eager = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I)
    for variant in range(3):
        lg = synth.logits(c, variant)
        xq, xs = mx.quantize_mx(synth.x(c, variant), mx.FMT_E4M3)
        lg_buf.copy_(dev(lg))
        xq_buf.copy_(dev(xq))
        xs_buf.copy_(dev(xs))
        g.replay()
        torch.cuda.synchronize()
        got = host(out_buf).copy()
        eager = moe.moe_layer(dev(lg), dev(xq), dev(xs), w1, w2, c.k, c.e0, c.n_local, ws=ws_eager)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got, host(eager))
        np.testing.assert_array_equal(host(ws.view("counts")), host(ws_eager.view("counts")))
        assert np.count_nonzero(got) > 0
