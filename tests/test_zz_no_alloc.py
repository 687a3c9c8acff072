"""moe_layer_noalloc (the layer with the library's fixed per-GPU workspace)
against moe_layer (caller workspace), through the C ABI (GPU): identical
kernels, so identical bits, on two calls in a row, the second with fewer
tokens than the first (the fixed array then still holds the first call's
larger intermediates)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("routed_grouped_gemm_amd")
from gpu_util import banner, host  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name,Ts", [("decode", (128, 8)), ("shared", (32, 5)), ("tiny", (16, 3))])
def test_noalloc_matches_workspace_entry(name, Ts):
    from dataclasses import replace
    from synth import device
    c0 = synth.config(name, Ts[0] if name == "decode" else None)
    dw = device.build_weights(c0)
    for T in Ts:
        c = replace(c0, T=T)
        banner(f"noalloc {name} T={T}")
        logits, xq, xs = device.build_inputs(c)
        ref = moe.moe_layer(logits, xq, xs, dw.w1, dw.w2, c.k, c.e0, c.n_local, dw.shared)
        out = torch.full((c.T, c.H), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.uint16)
        got = moe.moe_layer_noalloc(logits, xq, xs, dw.w1, dw.w2, c.k, c.e0, c.n_local, dw.shared, out=out)
        assert got.data_ptr() == out.data_ptr()
        np.testing.assert_array_equal(host(got), host(ref))
        assert np.any(host(ref) != 0)
