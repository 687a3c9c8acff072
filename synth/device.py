"""Device-side assembly of a synthetic workload for the GPU tests and the
benchmark: draws the float32 arrays from `synth`, uploads them, and quantises
and prepacks them with the library's own entry points (moe_quantize_mx,
moe_prepack_weights). Holds none of the method's arithmetic."""
from __future__ import annotations

from dataclasses import dataclass
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import routed_grouped_gemm_amd as moe
import synth


def fmt_code(w_fmt: str) -> int:
    return moe.MOE_FMT_MXFP4 if w_fmt == "e2m1" else moe.MOE_FMT_MXFP8


@dataclass
class DeviceWeights:
    w1: moe.PackedWeights
    w2: moe.PackedWeights
    shared: tuple | None


def _quant(arr: np.ndarray, fmt: int, device):
    t = torch.from_numpy(arr).to(device)
    return moe.moe_quantize_mx(t, fmt)


def build_weights(c: synth.Config, device="cuda", workers: int = 8) -> DeviceWeights:
    """Quantise + prepack every local expert's W1 and W2 (and the shared
    expert), one expert at a time; host draws run in a small thread pool."""
    fmt = fmt_code(c.w_fmt)
    w1 = moe.PackedWeights.empty(c.n_local, 2 * c.I, c.H, fmt, True, device)
    w2 = moe.PackedWeights.empty(c.n_local, c.H, c.I, fmt, False, device)

    def draw(g):
        return synth.w1(c, g), synth.w2(c, g)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        for g, (a, b) in enumerate(ex.map(draw, range(c.n_local))):
            q, s = _quant(a, fmt, device)
            w1.fill_group(g, q, s)
            q, s = _quant(b, fmt, device)
            w2.fill_group(g, q, s)
    shared = None
    if c.shared:
        sw1 = moe.PackedWeights.empty(1, 2 * c.I, c.H, fmt, True, device)
        sw2 = moe.PackedWeights.empty(1, c.H, c.I, fmt, False, device)
        q, s = _quant(synth.shared_w1(c), fmt, device)
        sw1.fill_group(0, q, s)
        q, s = _quant(synth.shared_w2(c), fmt, device)
        sw2.fill_group(0, q, s)
        shared = (sw1, sw2)
    torch.cuda.synchronize()
    return DeviceWeights(w1, w2, shared)


def build_inputs(c: synth.Config, variant: int = 0, device="cuda"):
    """Router logits (f32) and quantised activations for one routing draw."""
    logits = torch.from_numpy(synth.logits(c, variant)).to(device)
    xq, xs = _quant(synth.x(c, variant), moe.MOE_FMT_MXFP8, device)
    return logits, xq, xs
