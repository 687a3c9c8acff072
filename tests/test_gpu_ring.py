"""The token ring (MOE_LAYER_TOKEN_RING) against the call without it (GPU):
the producer copies the grouped token rows into ring slots on a second
stream and W1 consumes them chunk by chunk, so every output and intermediate
must be identical bit for bit (the arithmetic is the same, only where the
token rows are read from differs), including a case of three chunks over two
slots (each slot refilled after its chunk was consumed); one case is also
compared with the oracle."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import moe as omoe, mx
import synth

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("routed_grouped_gemm_amd")
from gpu_util import assert_layer_close, banner, bf16_bits, host  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(c, flags, dw, ins):
    logits, xq, xs = ins
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I, c.shared, flags)
    hT = (None, None)
    if c.transpose:
        ld = moe.moe_transposed_ld(c.R_max, c.G)
        hT = (torch.zeros((c.I, ld), dtype=torch.uint8, device="cuda"),
              torch.zeros((c.I, ld // 32), dtype=torch.uint8, device="cuda"))
    out = moe.moe_layer(logits, xq, xs, dw.w1, dw.w2, c.k, c.e0, c.n_local, dw.shared, flags, ws=ws,
                        hTq=hT[0], hTs=hT[1])
    R = int(host(ws.view("offsets"))[-1])
    res = [host(out), host(ws.view("hq"))[:R], host(ws.view("hs"))[:R], host(ws.view("y"))[:R]]
    if c.transpose:
        res += [host(hT[0]), host(hT[1])]
    return res


RING = [
    # 34 000 rows: about 141 passes of 256 rows, 3 chunks of 64 over 2 slots
    ("three-chunks", dict(T=17000, H=512, I=256, E=8, k=2, n_local=8, w_fmt="e4m3", transpose=True,
                          logit_kind="zipf"), True),
    ("prefill", dict(), False),
]


@pytest.mark.parametrize("name,kw,with_oracle", RING, ids=[r[0] for r in RING])
def test_ring_identical_to_direct(name, kw, with_oracle):
    from synth import device
    c = replace(synth.config("prefill"), **kw)
    banner(f"token ring {name} T={c.T} H={c.H} I={c.I} E={c.E} k={c.k}")
    dw = device.build_weights(c)
    ins = device.build_inputs(c)
    flags = moe.MOE_W1_WRITE_TRANSPOSE if c.transpose else 0
    direct = _run(c, flags, dw, ins)
    ring = _run(c, flags | moe.MOE_LAYER_TOKEN_RING, dw, ins)
    for i, (a, b) in enumerate(zip(direct, ring)):
        assert np.array_equal(a, b), f"result {i} differs between the ring and the direct call"
    if with_oracle:
        lg = synth.logits(c)
        xq, xs = mx.quantize_mx(synth.x(c), mx.FMT_E4M3)
        np.testing.assert_array_equal(host(ins[1]), xq)
        w1 = [mx.quantize_mx(synth.w1(c, g), c.w_fmt) for g in range(c.n_local)]
        w2 = [mx.quantize_mx(synth.w2(c, g), c.w_fmt) for g in range(c.n_local)]
        ref = omoe.moe_layer(lg, xq, xs, c.k, [q for q, _ in w1], [s for _, s in w1], [q for q, _ in w2],
                             [s for _, s in w2], c.w_fmt, c.I, n_local=c.n_local, transpose=c.transpose)
        assert_layer_close(ring[0], ref.out, "out (ring)")
