"""Whole-layer parity of moe_layer against the oracle (GPU).

Small shapes: every element, every intermediate, with the oracle's quantised
inputs uploaded to the GPU. Full workload sizes, called exactly as the
benchmark calls them: routing, counts and offsets for every token, and the
outputs of sampled tokens, which the oracle computes one by one from its own
quantisation of the same float32 draws (checked equal to the library's
quantisation of those draws first, so no oracle input comes from the GPU).
"""
from dataclasses import replace

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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _oracle_inputs(c, variant=0):
    lg = synth.logits(c, variant)
    xq, xs = mx.quantize_mx(synth.x(c, variant), mx.FMT_E4M3)
    w1 = [mx.quantize_mx(synth.w1(c, g), c.w_fmt) for g in range(c.n_local)]
    w2 = [mx.quantize_mx(synth.w2(c, g), c.w_fmt) for g in range(c.n_local)]
    sh = None
    if c.shared:
        a, b = mx.quantize_mx(synth.shared_w1(c), c.w_fmt), mx.quantize_mx(synth.shared_w2(c), c.w_fmt)
        sh = (a[0], a[1], b[0], b[1])
    return lg, xq, xs, w1, w2, sh


def _packed(ws, fmt, is_w1):
    return moe.PackedWeights(dev(np.stack([a[0] for a in ws])), dev(np.stack([a[1] for a in ws])),
                             FMT[fmt], is_w1)


SMALL = [
    ("tiny", dict(), 0),
    ("mid-share", dict(T=40, H=1024, I=512, E=32, k=4, e0=8, n_local=12, shared=True), 0),
    ("mxfp8-transpose", dict(T=300, H=512, I=384, E=8, k=2, n_local=8, w_fmt="e4m3",
                             transpose=True), moe.MOE_W1_WRITE_TRANSPOSE),
    ("renorm-ceil", dict(T=24, E=16, k=4, n_local=16), moe.MOE_ROUTE_RENORM | moe.MOE_SCALE_RULE_CEIL),
    ("weight-at-combine", dict(T=20, E=8, k=3, n_local=8), moe.MOE_WEIGHT_AT_COMBINE),
    ("ragged-passes", dict(T=200, H=768, I=256, E=4, k=2, n_local=4, shared=True), 0),
    # at most 8 tokens: the W1 launch routes and groups the tokens itself
    ("self-route-renorm-ceil", dict(T=6, E=16, k=4, n_local=16), moe.MOE_ROUTE_RENORM | moe.MOE_SCALE_RULE_CEIL),
    ("self-route-shared-wc", dict(T=5, H=1024, I=512, E=32, k=4, e0=8, n_local=12, shared=True),
     moe.MOE_WEIGHT_AT_COMBINE),
    ("self-route-one-token", dict(T=1, E=64, k=8, e0=16, n_local=24), 0),
    # at most 16 tokens on at most 4 expected active groups (the one-token
    # case above, single-expert, every-expert): W2 and the combine run as
    # one launch; 16 tokens over 2 local experts and the shared one fill
    # whole 16-row tiles in it; the same cases with the separate W2 and
    # combine launches forced
    ("w2-combine-full-tiles", dict(T=16, E=2, k=2, n_local=2, shared=True), moe.MOE_WEIGHT_AT_COMBINE),
    ("w2-combine-full-tiles-separate", dict(T=16, E=2, k=2, n_local=2, shared=True),
     moe.MOE_WEIGHT_AT_COMBINE | moe.MOE_LAYER_SEPARATE_KERNELS),
    ("self-route-one-token-separate", dict(T=1, E=64, k=8, e0=16, n_local=24), moe.MOE_LAYER_SEPARATE_KERNELS),
    # degenerate routing: one expert (every weight exactly 1), and k = E
    # (every token picks every expert)
    ("single-expert", dict(T=7, E=1, k=1, n_local=1), 0),
    ("every-expert", dict(T=9, E=4, k=4, n_local=4), 0),
    # about 275 rows per expert: the LDS-tiled GEMMs, with the transposed copy
    ("tiled-mxfp8-transpose", dict(T=1100, H=512, I=384, E=8, k=2, n_local=8, w_fmt="e4m3",
                                   transpose=True), moe.MOE_W1_WRITE_TRANSPOSE),
]


@pytest.mark.parametrize("name,kw,flags", SMALL, ids=[s[0] for s in SMALL])
def test_layer_small_every_element(name, kw, flags):
    c = replace(synth.config("tiny"), **kw)
    banner(f"layer {name} {c}")
    lg, xq, xs, w1, w2, sh = _oracle_inputs(c)
    rule = "ceil" if flags & moe.MOE_SCALE_RULE_CEIL else "ocp"
    ref = omoe.moe_layer(lg, xq, xs, c.k, [a[0] for a in w1], [a[1] for a in w1], [a[0] for a in w2],
                         [a[1] for a in w2], c.w_fmt, c.I, e0=c.e0, n_local=c.n_local, shared=sh,
                         renorm=bool(flags & moe.MOE_ROUTE_RENORM),
                         transpose=bool(flags & moe.MOE_W1_WRITE_TRANSPOSE),
                         weight_at_combine=bool(flags & moe.MOE_WEIGHT_AT_COMBINE), rule=rule)
    pw1, pw2 = _packed(w1, c.w_fmt, True), _packed(w2, c.w_fmt, False)
    shared = None
    if sh is not None:
        shared = (moe.PackedWeights(dev(sh[0][None]), dev(sh[1][None]), FMT[c.w_fmt], True),
                  moe.PackedWeights(dev(sh[2][None]), dev(sh[3][None]), FMT[c.w_fmt], False))
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I, c.shared, flags)
    hTq = hTs = None
    if flags & moe.MOE_W1_WRITE_TRANSPOSE:
        ld = moe.moe_transposed_ld(c.R_max, c.G)
        hTq = torch.zeros((c.I, ld), dtype=torch.uint8, device="cuda")
        hTs = torch.zeros((c.I, ld // 32), dtype=torch.uint8, device="cuda")
    out = moe.moe_layer(dev(lg), dev(xq), dev(xs), pw1, pw2, c.k, c.e0, c.n_local, shared, flags,
                        ws=ws, hTq=hTq, hTs=hTs)
    R = int(ref.perm.offsets[-1])
    np.testing.assert_array_equal(host(ws.view("topk_idx")), ref.topk_idx)
    np.testing.assert_allclose(host(ws.view("topk_w")), ref.topk_w, rtol=1e-5)
    np.testing.assert_array_equal(host(ws.view("counts")), ref.perm.counts)
    np.testing.assert_array_equal(host(ws.view("offsets")), ref.perm.offsets)
    np.testing.assert_array_equal(host(ws.view("slot_row")), ref.perm.slot_row)
    np.testing.assert_array_equal(host(ws.view("row_src"))[:R], ref.perm.row_src)
    # h: one E4M3 step plus the propagated accumulation bound
    xq_p, xs_p = omoe.gather_rows(xq, xs, ref.perm)
    X = np.abs(mx.dequantize_mx(xq_p, xs_p, mx.FMT_E4M3))
    ws1 = [a for a in w1] + ([(sh[0], sh[1])] if sh else [])
    mag = np.zeros_like(ref.w1.acc)
    for g in range(c.G):
        lo, hi = ref.perm.offsets[g], ref.perm.offsets[g + 1]
        if hi > lo:
            mag[lo:hi] = X[lo:hi] @ np.abs(mx.dequantize_mx(ws1[g][0], ws1[g][1], c.w_fmt)).T
    wts = np.ones(R) if flags & moe.MOE_WEIGHT_AT_COMBINE else ref.perm.row_w
    gate, up = ref.w1.acc[:, :c.I], ref.w1.acc[:, c.I:]
    dg, du = MFMA_REL * mag[:, :c.I], MFMA_REL * mag[:, c.I:]
    dh = (1.1 * (np.abs(up) + du) * dg + np.abs(omoe.silu(gate)) * du) * np.abs(wts)[:, None] \
        + 2e-5 * np.abs(ref.w1.h)                         # fp32 routing weight vs fp64
    assert_mx_within_1ulp(host(ws.view("hq"))[:R], host(ws.view("hs"))[:R], ref.w1.hq, ref.w1.hs,
                          "h", extra_tol=dh)
    if flags & moe.MOE_W1_WRITE_TRANSPOSE:
        q_ref, s_ref = omoe.concat_transposed(ref.w1.hTq, ref.w1.hTs, c.I)
        n = q_ref.shape[1]
        assert_mx_within_1ulp(host(hTq)[:, :n], host(hTs)[:, :n // 32], q_ref, s_ref, "hT",
                              max_frac_diff=0.02, extra_tol=_transpose_tol(dh, ref, c))
    assert_layer_close(bf16_bits(out), ref.out, "out")


def test_layer_no_tokens():
    """T = 0: a valid call that enqueues nothing and returns an empty output."""
    c = replace(synth.config("tiny"), T=1)
    _, _, _, w1, w2, _ = _oracle_inputs(c)
    pw1, pw2 = _packed(w1, c.w_fmt, True), _packed(w2, c.w_fmt, False)
    lg = torch.empty((0, c.E), dtype=torch.float32, device="cuda")
    xq = torch.empty((0, c.H), dtype=torch.uint8, device="cuda")
    xs = torch.empty((0, c.H // 32), dtype=torch.uint8, device="cuda")
    out = moe.moe_layer(lg, xq, xs, pw1, pw2, c.k, c.e0, c.n_local)
    assert tuple(out.shape) == (0, c.H)


@pytest.mark.parametrize("T", [1, 3])
def test_layer_no_local_rows(T):
    """No token picks a local expert: the GEMMs have no work item, and every
    output element must still be written, as an exact zero, over a buffer
    that held NaNs."""
    c = replace(synth.config("tiny"), T=T, E=64, k=2, n_local=4)
    lg = synth.logits(c)
    picked = set(omoe.route(lg, c.k)[0].ravel().tolist())
    e0 = next(e for e in range(0, c.E - c.n_local + 1) if not picked & set(range(e, e + c.n_local)))
    c = replace(c, e0=e0)
    banner(f"layer without local rows {c}")
    _, xq, xs, w1, w2, _ = _oracle_inputs(c)
    pw1, pw2 = _packed(w1, c.w_fmt, True), _packed(w2, c.w_fmt, False)
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I)
    out = torch.full((c.T, c.H), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.uint16)   # BF16 NaN
    moe.moe_layer(dev(lg), dev(xq), dev(xs), pw1, pw2, c.k, c.e0, c.n_local, out=out, ws=ws)
    assert host(ws.view("counts")).sum() == 0
    np.testing.assert_array_equal(host(out), np.zeros((c.T, c.H), np.uint16))


def _transpose_tol(dh, ref, c):
    n = sum((int(ref.perm.counts[g]) + 31) // 32 * 32 for g in range(c.G))
    t = np.zeros((c.I, n))
    col = 0
    for g in range(c.G):
        lo, hi = ref.perm.offsets[g], ref.perm.offsets[g + 1]
        t[:, col:col + hi - lo] = dh[lo:hi].T
        col += (hi - lo + 31) // 32 * 32
    return t


# ---------------------------------------------------------------- full size
_WEIGHTS = {}
_EXPERTS = {}           # (seed, fmt, H, I, g) -> oracle codes (w1q, w1s, w2q, w2s); g = -1: shared


def _device_weights(c):
    from synth import device
    key = (c.seed, c.w_fmt, c.n_local, c.H, c.I, c.shared)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        torch.cuda.empty_cache()
        _WEIGHTS[key] = device.build_weights(c)
    return _WEIGHTS[key]


def _experts(c, gs):
    """The oracle's own quantisation of experts gs (-1: the shared expert),
    drawn from the same float32 arrays the GPU weights were made from; the
    library's quantisation of those arrays is checked byte-identical, so the
    GPU computes on exactly the oracle's inputs. Prepared in parallel host
    threads (NumPy releases the interpreter lock), cached per weight set."""
    from concurrent.futures import ThreadPoolExecutor
    base = (c.seed, c.w_fmt, c.H, c.I)
    if any(k[:4] != base for k in _EXPERTS):
        _EXPERTS.clear()
    need = sorted({g for g in gs if base + (g,) not in _EXPERTS})

    def draw(g):
        a32 = synth.shared_w1(c) if g < 0 else synth.w1(c, g)
        b32 = synth.shared_w2(c) if g < 0 else synth.w2(c, g)
        return g, a32, b32, mx.quantize_mx(a32, c.w_fmt), mx.quantize_mx(b32, c.w_fmt)

    with ThreadPoolExecutor(max_workers=16) as ex:
        for i in range(0, len(need), 16):
            for g, a32, b32, (qa, sa), (qb, sb) in ex.map(draw, need[i:i + 16]):
                gq, gsc = moe.moe_quantize_mx(dev(a32), FMT[c.w_fmt])
                assert np.array_equal(host(gq), qa) and np.array_equal(host(gsc), sa), f"W1[{g}] quantisation"
                gq, gsc = moe.moe_quantize_mx(dev(b32), FMT[c.w_fmt])
                assert np.array_equal(host(gq), qb) and np.array_equal(host(gsc), sb), f"W2[{g}] quantisation"
                _EXPERTS[base + (g,)] = (qa, sa, qb, sb)
    return {g: _EXPERTS[base + (g,)] for g in gs}


def _pick_tokens(c, perm, rng, n=16, budget=48):
    """n tokens with a local slot, spread over the rows (and so the passes) of
    the largest group, the rest drawn at random; a token is taken while the
    distinct local experts of the picks stay within `budget` (the oracle
    prepares every expert a pick uses)."""
    k = c.k
    gl = int(np.argmax(perm.counts[:c.n_local]))
    lo, hi = int(perm.offsets[gl]), int(perm.offsets[gl + 1])
    spread = [int(perm.row_src[r]) for r in np.linspace(lo, hi - 1, num=min(8, hi - lo)).astype(int)]
    local = perm.slot_row[:, :k] >= 0
    cand = list(dict.fromkeys(spread + list(rng.permutation(np.flatnonzero(local.any(1))))))
    picks, experts = [], set()
    for t in cand:
        es = _local_groups(perm, t, k)
        if len(experts | es) <= budget:
            picks.append(int(t))
            experts |= es
        if len(picks) == n:
            break
    return picks


def _local_groups(perm, t, k):
    """Local groups of token t's routed slots (from the oracle's grouping)."""
    rows = perm.slot_row[t, :k]
    return {int(np.searchsorted(perm.offsets, r, side="right") - 1) for r in rows if r >= 0}


def _check_group(c, g, w, ws, perm, x32, xq_d, xs_d, hT):
    """Every element of group g's h (codes, scales), transposed copy and y
    rows against the oracle, computed from the oracle's own quantisation of
    the group's token rows and weights."""
    lo, hi = int(perm.offsets[g]), int(perm.offsets[g + 1])
    n = hi - lo
    if n == 0:
        return
    print(f"  whole group {g}: {n} rows", flush=True)
    src = perm.row_src[lo:hi]
    xq_g, xs_g = mx.quantize_mx(x32[src], mx.FMT_E4M3)
    np.testing.assert_array_equal(host(xq_d)[src], xq_g)
    np.testing.assert_array_equal(host(xs_d)[src], xs_g)
    w1q, w1s, w2q, w2s = w
    loc = np.array([0, n], np.int32)
    o1 = omoe.grouped_w1(xq_g, xs_g, loc, perm.row_w[lo:hi], [w1q], [w1s], c.w_fmt, c.I,
                         transpose=c.transpose)
    X = np.abs(mx.dequantize_mx(xq_g, xs_g, mx.FMT_E4M3))
    mag = X @ np.abs(mx.dequantize_mx(w1q, w1s, c.w_fmt)).T
    gate, up = o1.acc[:, :c.I], o1.acc[:, c.I:]
    dg, du = MFMA_REL * mag[:, :c.I], MFMA_REL * mag[:, c.I:]
    wts = np.abs(perm.row_w[lo:hi])[:, None]
    dh = (1.1 * (np.abs(up) + du) * dg + np.abs(omoe.silu(gate)) * du) * wts + 2e-5 * np.abs(o1.h)
    hq_g, hs_g = host(ws.view("hq"))[lo:hi], host(ws.view("hs"))[lo:hi]
    assert_mx_within_1ulp(hq_g, hs_g, o1.hq, o1.hs, f"group {g} h", extra_tol=dh)
    if c.transpose:
        off32 = np.zeros(c.G + 1, np.int64)
        off32[1:] = np.cumsum((perm.counts.astype(np.int64) + 31) // 32 * 32)
        n32 = (n + 31) // 32 * 32
        c0 = int(off32[g])
        tq = host(hT[0])[:, c0:c0 + n32]
        ts = host(hT[1])[:, c0 // 32:(c0 + n32) // 32]
        dT = np.zeros((c.I, n32))
        dT[:, :n] = dh.T
        assert_mx_within_1ulp(tq, ts, o1.hTq[0], o1.hTs[0], f"group {g} hT", extra_tol=dT)
    # y from the oracle's own h; the bound adds what the GPU's h deviates by
    # (within one E4M3 step, checked above) through |W2|
    y_ref = omoe.grouped_w2(o1.hq, o1.hs, loc, [w2q], [w2s], c.w_fmt, H=c.H)
    W2 = np.abs(mx.dequantize_mx(w2q, w2s, c.w_fmt))
    h_gpu = mx.dequantize_mx(hq_g, hs_g, mx.FMT_E4M3)
    mag_y = np.abs(h_gpu) @ W2.T
    dy = np.abs(h_gpu - mx.dequantize_mx(o1.hq, o1.hs, mx.FMT_E4M3)) @ W2.T + MFMA_REL * mag_y
    assert_bf16_close(bf16_bits(ws.view("y"))[lo:hi], y_ref, f"group {g} y", max_ulp=1, abs_floor=dy,
                      mag=mag_y)
    assert_layer_close(bf16_bits(ws.view("y"))[lo:hi], y_ref, f"group {g} y")


@pytest.mark.parametrize("T", [8, 16, 32, 48])
def test_layer_routing_ties(T):
    """Routing and grouping with tied logits on the routers inside the
    layer: W1's own routing at T = 8 of the decode share (8-wave items, a
    whole wave per token) and at T = 16 (4-wave items, 16 lanes per token),
    and the one-workgroup router and grouping (16 lanes per token) at T = 32
    and 48; every selection, weight, count, offset and row bit-exact against
    the oracle (weights to 1e-5)."""
    from synth import device
    c = synth.config("decode", T)
    banner(f"layer routing ties T={T} E={c.E} k={c.k} local={c.n_local}")
    dw = _device_weights(c)
    _, xq_d, xs_d = device.build_inputs(c)
    lg = synth.logits(c).copy()
    lg[1, :] = np.float32(0.5)                           # all tied
    lg[2, 40:48] = lg[2].max() + 1                       # ties at the top
    lg[3, :] = -1.0                                      # -0 and +0 tie: the lower id first
    lg[3, 10:40:2] = -0.0
    lg[3, 11:41:2] = 0.0
    lg[5, 0:32] = lg[5].max() + 2                        # a tie across every local expert
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I, c.shared, 0)
    moe.moe_layer(dev(lg), xq_d, xs_d, dw.w1, dw.w2, c.k, c.e0, c.n_local, dw.shared, 0, ws=ws)
    idx_ref, w_ref = omoe.route(lg, c.k)
    np.testing.assert_array_equal(host(ws.view("topk_idx")), idx_ref)
    np.testing.assert_allclose(host(ws.view("topk_w")), w_ref, rtol=1e-5, atol=0)
    perm = omoe.permute(idx_ref, w_ref, c.e0, c.n_local, c.shared)
    R = int(perm.offsets[-1])
    np.testing.assert_array_equal(host(ws.view("counts")), perm.counts)
    np.testing.assert_array_equal(host(ws.view("offsets")), perm.offsets)
    np.testing.assert_array_equal(host(ws.view("slot_row")), perm.slot_row)
    np.testing.assert_array_equal(host(ws.view("row_src"))[:R], perm.row_src)


FULL = [("decode", 1), ("decode", 8), ("decode", 32), ("decode", 128), ("shared", None),
        ("full", None), ("prefill", None)]


@pytest.mark.parametrize("name,T", FULL, ids=[f"{n}-{t}" for n, t in FULL])
def test_layer_full_size_sampled(name, T):
    """The workload at its full size, launched as the benchmark launches it:
    routing and grouping of every token bit-exact; every element of whole
    groups (the largest, and the smallest non-empty one; the shared group)
    against the oracle; 16 sampled tokens' output rows, which the oracle
    computes one by one."""
    from synth import device
    c = synth.config(name, T)
    banner(f"full-size layer {name} T={c.T} H={c.H} I={c.I} E={c.E} k={c.k}")
    dw = _device_weights(c)
    logits, xq_d, xs_d = device.build_inputs(c)
    flags = moe.MOE_W1_WRITE_TRANSPOSE if c.transpose else 0
    ws = moe.LayerWorkspace(c.T, c.E, c.k, c.n_local, c.H, c.I, c.shared, flags)
    hTq = hTs = None
    if c.transpose:
        ld = moe.moe_transposed_ld(c.R_max, c.G)
        hTq = torch.empty((c.I, ld), dtype=torch.uint8, device="cuda")
        hTs = torch.empty((c.I, ld // 32), dtype=torch.uint8, device="cuda")
    out = moe.moe_layer(logits, xq_d, xs_d, dw.w1, dw.w2, c.k, c.e0, c.n_local, dw.shared, flags,
                        ws=ws, hTq=hTq, hTs=hTs)
    got = bf16_bits(out)

    # routing and grouping of every token
    lg = synth.logits(c)
    idx_ref, w_ref = omoe.route(lg, c.k)
    np.testing.assert_array_equal(host(ws.view("topk_idx")), idx_ref)
    perm = omoe.permute(idx_ref, w_ref, c.e0, c.n_local, c.shared)
    np.testing.assert_array_equal(host(ws.view("counts")), perm.counts)
    np.testing.assert_array_equal(host(ws.view("offsets")), perm.offsets)
    R = int(perm.offsets[-1])
    np.testing.assert_array_equal(host(ws.view("row_src"))[:R], perm.row_src)
    np.testing.assert_array_equal(host(ws.view("slot_row")), perm.slot_row)

    # whole groups, every element
    x32 = synth.x(c)
    cnt = perm.counts[:c.n_local]
    groups = [int(np.argmax(cnt))]
    if name in ("prefill", "full"):
        groups.append(int(np.flatnonzero(cnt == cnt[cnt > 0].min())[0]))
    wgt = {g: e for g, e in _experts(c, groups).items()}
    if c.shared:
        groups.append(c.n_local)
        wgt[c.n_local] = _experts(c, [-1])[-1]
    for g in groups:
        _check_group(c, g, wgt[g], ws, perm, x32, xq_d, xs_d, (hTq, hTs))

    # sampled tokens, computed one by one by the oracle
    rng = np.random.default_rng(c.T)
    picks = _pick_tokens(c, perm, rng, n=16, budget=64 if name == "prefill" else 40)
    local = (perm.slot_row[:, :c.k] >= 0).sum(1)
    none = np.flatnonzero(local == 0)
    if len(none) and not c.shared:
        picks.append(int(none[0]))                 # a token with no local slot: exact zeros
    gs = sorted(set().union(*[_local_groups(perm, t, c.k) for t in picks]))
    print(f"  {len(picks)} sampled tokens over {len(gs)} local experts", flush=True)
    ex = _experts(c, gs)
    sh = _experts(c, [-1])[-1] if c.shared else None
    xq_ref, xs_ref = mx.quantize_mx(x32[picks], mx.FMT_E4M3)
    np.testing.assert_array_equal(host(xq_d)[picks], xq_ref)
    np.testing.assert_array_equal(host(xs_d)[picks], xs_ref)
    ref_rows = np.stack([omoe.token_output(lg[t], xq_ref[i], xs_ref[i], c.k, ex.__getitem__, c.w_fmt, c.I,
                                           c.e0, c.n_local, sh) for i, t in enumerate(picks)])
    for i, t in enumerate(picks):
        if local[t] == 0 and not c.shared:
            assert np.all(got[t] == 0), f"token {t} has no local slot but a nonzero row"
        else:
            assert_layer_close(got[t], ref_rows[i], f"token {t} ({local[t]} local slots)")
    assert_layer_close(got[picks], ref_rows, f"{len(picks)} sampled tokens together")
