"""Stage-by-stage parity of the HIP path against the oracle (GPU).

Each kernel gets the oracle's inputs for its stage, through the C ABI, and its
outputs are compared with the oracle's outputs for that stage:
  quantise, route, permute: bit-exact (routing weights to 1e-5 relative)
  grouped W1: h codes within one E4M3 step (fp32 MFMA vs fp64 accumulation)
  grouped W2: y within one BF16 step plus the MFMA inner-sum error bound
  combine: bit-exact given the same y
"""
import numpy as np
import pytest
import torch

from oracle import moe as omoe, mx
import synth

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("routed_grouped_gemm_amd")
from gpu_util import (MFMA_REL, assert_bf16_close, assert_mx_within_1ulp, banner, bf16_bits,  # noqa: E402
                      dev, host)

FMT = {"e2m1": moe.MOE_FMT_MXFP4, "e4m3": moe.MOE_FMT_MXFP8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ------------------------------------------------------------------ quantise
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("rule", ["ocp", "ceil"])
def test_quantize_bit_exact(fmt, rule):
    banner(f"quantize {fmt} {rule}")
    rng = np.random.default_rng(21)
    v = (rng.standard_normal((96, 256)) * 10.0 ** rng.uniform(-8, 8, (96, 1))).astype(np.float32)
    v[0] = 0.0
    v[1, :] = 0.0
    v[1, 7] = -1e-40                                     # fp32 subnormal amax
    v[2] = np.round(v[2] / np.abs(v[2]).max() * 8) / 8 * 448   # exact ties after scaling
    v[3] = np.float32(1e38) * np.sign(rng.standard_normal(256))
    v[4, ::2] = -0.0
    q_ref, s_ref = mx.quantize_mx(v.astype(np.float64), fmt, rule)
    flags = moe.MOE_SCALE_RULE_CEIL if rule == "ceil" else 0
    q, s = moe.moe_quantize_mx(dev(v), FMT[fmt], flags)
    np.testing.assert_array_equal(host(s), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)


# --------------------------------------------------------------------- route
ROUTE_CASES = [
    ("tiny", None, 0), ("decode", 128, 0), ("decode", 1, 0), ("full", None, 0), ("prefill", None, 0),
    ("tiny", None, moe.MOE_ROUTE_RENORM),
]


@pytest.mark.parametrize("name,T,flags", ROUTE_CASES)
def test_route_parity(name, T, flags):
    c = synth.config(name, T)
    banner(f"route {name} T={c.T} E={c.E} k={c.k} flags={flags}")
    lg = synth.logits(c)
    if c.T > 4:
        lg[1, :] = np.float32(0.5)                       # all tied
        lg[2, 5:9] = lg[2, 5:9].max() + 1                # ties at the top
        lg[3, :] = -1.0                                  # -0 and +0 tie: the lower id first
        lg[3, 10:20:2] = -0.0
        lg[3, 11:21:2] = 0.0
    idx_ref, w_ref = omoe.route(lg, c.k, renorm=bool(flags & moe.MOE_ROUTE_RENORM))
    idx, w = moe.moe_route(dev(lg), c.k, flags)
    np.testing.assert_array_equal(host(idx), idx_ref)
    np.testing.assert_allclose(host(w), w_ref, rtol=1e-5, atol=0)


@pytest.mark.parametrize("T,E,k", [(37, 100, 16), (70, 33, 3), (5, 256, 16)])
def test_route_parity_lane_edges(T, E, k):
    """Expert counts that leave the last lanes of a token's lane group partly
    or wholly past E, and top-16 (as many selections as half a lane group);
    ties as in test_route_parity."""
    banner(f"route lane edges T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 1000 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[1, :] = np.float32(0.25)                          # all tied
    lg[2, E // 2:E // 2 + 4] = lg[2].max() + 1           # ties at the top
    lg[3, :] = -1.0                                      # -0 and +0 tie: the lower id first
    lg[3, 1:E:3] = -0.0
    lg[3, 2:E:3] = 0.0
    for flags in (0, moe.MOE_ROUTE_RENORM):
        idx_ref, w_ref = omoe.route(lg, k, renorm=bool(flags & moe.MOE_ROUTE_RENORM))
        idx, w = moe.moe_route(dev(lg), k, flags)
        np.testing.assert_array_equal(host(idx), idx_ref)
        np.testing.assert_allclose(host(w), w_ref, rtol=1e-5, atol=0)


# ------------------------------------------------------------------- permute
PERMUTE_CASES = [
    # T, E, k, e0, n_local, shared, H
    (16, 8, 2, 0, 8, False, 512),           # single-workgroup path
    (128, 256, 8, 0, 32, False, 7168),      # decode share
    (32, 256, 8, 64, 32, True, 1024),       # other share + shared expert
    (1, 256, 8, 0, 32, False, 256),         # likely no local slot
    (16384, 64, 6, 0, 64, False, 256),      # chunked path (count / scan / scatter)
    (700, 2048, 8, 0, 2048, True, 256),     # many experts, chunked
    (4000, 16, 1, 3, 10, True, 512),        # k = 1, partial share, single workgroup at the edge
    # at most 256 assignments and 64 groups: one wave does the whole grouping
    (8, 256, 8, 0, 32, True, 512),          # 64 assignments: one per lane, with a shared expert
    (16, 64, 8, 0, 40, False, 256),         # 128 assignments: two per lane
    (30, 32, 4, 5, 20, True, 256),          # 120 assignments, partial share
    (31, 256, 8, 0, 64, False, 256),        # 248 assignments over 64 groups
    # past the one-wave limits: the workgroup path
    (100, 64, 6, 0, 50, True, 256),         # 600 assignments, shared expert
    (128, 128, 8, 0, 63, True, 256),        # 1024 assignments, 64 groups
    (33, 16, 8, 3, 13, False, 256),         # 264 assignments: just past 256
    (3, 16, 4, 2, 13, True, 256),           # partial share
    (64, 4, 1, 0, 4, False, 256),           # k = 1, 64 tokens
    (5, 64, 8, 0, 63, True, 256),           # 64 groups, the limit
    (2, 1, 1, 0, 1, True, 256),             # one routed expert (no group bits)
]


@pytest.mark.parametrize("T,E,k,e0,nl,sh,H", PERMUTE_CASES)
def test_permute_parity(T, E, k, e0, nl, sh, H):
    banner(f"permute T={T} E={E} k={k} e0={e0} nl={nl} shared={sh} H={H}")
    rng = np.random.default_rng(T + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = omoe.route(lg, k)
    w32 = w.astype(np.float32)
    ref = omoe.permute(idx, w32.astype(np.float64), e0, nl, sh)
    xq = rng.integers(0, 256, (T, H), dtype=np.uint8)
    xs = rng.integers(100, 150, (T, H // 32), dtype=np.uint8)
    out = moe.moe_permute(dev(idx), dev(w32), e0, nl, sh, dev(xq), dev(xs))
    R = int(ref.offsets[-1])
    np.testing.assert_array_equal(host(out["counts"]), ref.counts)
    np.testing.assert_array_equal(host(out["offsets"]), ref.offsets)
    np.testing.assert_array_equal(host(out["offsets32"])[1:] - host(out["offsets32"])[:-1],
                                  (ref.counts + 31) // 32 * 32)
    np.testing.assert_array_equal(host(out["row_src"])[:R], ref.row_src)
    np.testing.assert_array_equal(host(out["row_w"])[:R], ref.row_w.astype(np.float32))
    np.testing.assert_array_equal(host(out["slot_row"]), ref.slot_row)
    xq_ref, xs_ref = omoe.gather_rows(xq, xs, ref)
    np.testing.assert_array_equal(host(out["xq_perm"])[:R], xq_ref)
    np.testing.assert_array_equal(host(out["xs_perm"])[:R], xs_ref)


# ---------------------------------------------------------- grouped GEMMs
def _grouped_problem(counts, H, I, w_fmt, seed):
    """Oracle-made inputs of the grouped stages with chosen rows per group."""
    c = synth.Config("stage", 1, H, I, len(counts), 1, 0, len(counts), w_fmt, "normal", seed=seed)
    rng = np.random.default_rng(seed)
    G = len(counts)
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    xq, xs = mx.quantize_mx(rng.standard_normal((R, H)), mx.FMT_E4M3)
    row_w = rng.uniform(0.05, 1.0, R).astype(np.float32)
    w1 = [mx.quantize_mx(synth.w1(c, g), w_fmt) for g in range(G)]
    w2 = [mx.quantize_mx(synth.w2(c, g), w_fmt) for g in range(G)]
    return offsets, xq, xs, row_w, w1, w2


def _packed(ws, fmt, is_w1):
    q = np.stack([a[0] for a in ws])
    s = np.stack([a[1] for a in ws])
    return moe.PackedWeights(dev(q), dev(s), FMT[fmt], is_w1)


W1_CASES = [
    # counts, H, I, fmt, flags  (flags bit 31: read the token rows through row_src)
    ([0, 1, 17, 70, 33, 5], 1024, 512, "e2m1", 0),
    ([2, 0, 40, 9], 1024, 256, "e2m1", 1 << 31),
    ([64, 3], 512, 256, "e4m3", (1 << 31) | moe.MOE_W1_WRITE_TRANSPOSE),
    ([3, 0, 64, 129], 512, 256, "e4m3", 0),
    ([45, 0, 100, 32, 1], 512, 384, "e4m3", moe.MOE_W1_WRITE_TRANSPOSE),
    ([7, 90], 768, 256, "e2m1", moe.MOE_SCALE_RULE_CEIL | moe.MOE_W1_WRITE_TRANSPOSE),
    ([5, 12, 0, 40], 512, 256, "e2m1", moe.MOE_WEIGHT_AT_COMBINE),
    # several 256-row passes, ragged tails, empty groups
    ([0, 1, 255, 256, 257, 600, 33], 512, 256, "e4m3", (1 << 31) | moe.MOE_W1_WRITE_TRANSPOSE),
    ([300, 17, 513], 1024, 512, "e2m1", 0),
    ([520, 0, 64], 512, 384, "e4m3", moe.MOE_SCALE_RULE_CEIL | moe.MOE_W1_WRITE_TRANSPOSE),
    # last passes of exactly 128 and of 129 rows (in a pass of at most 128
    # rows the LDS-tiled kernel's second token half skips its work)
    ([128, 384, 0, 129, 640, 1], 512, 256, "e4m3", moe.MOE_W1_WRITE_TRANSPOSE),
    # 16 weight tiles (I = 2048) x about 50 row passes: about 800 work items,
    # so each workgroup of the LDS-tiled kernel's persistent grid walks three
    # or four of them (the cross-item prefetch, the stage reused as epilogue
    # scratch); ragged tails and an empty group, with the transposed copy
    ([5000, 257, 0, 3100, 2555, 1031], 512, 2048, "e4m3", (1 << 31) | moe.MOE_W1_WRITE_TRANSPOSE),
    ([4100, 6000, 1, 1955], 256, 2048, "e2m1", moe.MOE_SCALE_RULE_CEIL),
    # a long K (64 K-tiles): the pass-resident kernel stages its token rows in
    # K-chunks, double-buffered (32- and 64-row passes do not fit whole)
    ([40, 0, 70, 5, 33], 8192, 256, "e2m1", 1 << 31),
    ([23, 66, 130], 8192, 128, "e4m3", moe.MOE_W1_WRITE_TRANSPOSE),
    # 32 active groups x 64 units (I = 2048): 2048 work items, where every
    # K split ties and the decode kernel takes two waves per workgroup
    ([(7 * g) % 16 + 1 for g in range(32)], 1024, 2048, "e2m1", 1 << 31),
]

# The kernel family, forced by a flag: the weight-streaming kernel (weights
# streamed once, K split across waves), the pass-resident streaming kernel
# (a pass of token rows staged once, each weight unit over the whole K by one
# wave; 32-row passes with the transposed copy) or the LDS-tiled kernel
# (256 x 256 workgroup tiles). All must give the same answers.
KERNELS = {"decode": moe.MOE_GEMM_STREAMED, "pass": moe.MOE_GEMM_PASS, "tiled": moe.MOE_GEMM_TILED}


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("counts,H,I,fmt,flags", W1_CASES)
def test_grouped_w1_parity(counts, H, I, fmt, flags, kernel):
    banner(f"grouped_w1 {kernel} counts={counts} H={H} I={I} fmt={fmt} flags={flags}")
    gather = bool(flags & (1 << 31))
    flags &= ~(1 << 31)
    offsets, xq, xs, row_w, w1, _ = _grouped_problem(counts, H, I, fmt, 5 + H + I)
    G = len(counts)
    R = int(offsets[-1])
    row_src = None
    if gather:
        # the grouped rows are token rows picked through row_src from a token array
        rng = np.random.default_rng(R)
        T = max(R // 2, 1)
        tq, ts = mx.quantize_mx(rng.standard_normal((T, H)), mx.FMT_E4M3)
        row_src = rng.integers(0, T, R).astype(np.int32)
        xq, xs = tq[row_src], ts[row_src]
    rule = "ceil" if flags & moe.MOE_SCALE_RULE_CEIL else "ocp"
    wts = np.ones(R) if flags & moe.MOE_WEIGHT_AT_COMBINE else row_w.astype(np.float64)
    transpose = bool(flags & moe.MOE_W1_WRITE_TRANSPOSE)
    ref = omoe.grouped_w1(xq, xs, offsets, wts, [a[0] for a in w1], [a[1] for a in w1], fmt, I,
                          transpose=transpose, rule=rule)
    pw = _packed(w1, fmt, True)
    counts_d = dev(np.array(counts, np.int32))
    off32 = np.zeros(G + 1, np.int32)
    off32[1:] = np.cumsum((np.array(counts) + 31) // 32 * 32)
    kflags = flags | KERNELS[kernel]
    if gather:
        hq, hs, hTq, hTs = moe.moe_grouped_w1(pw, counts_d, dev(offsets), dev(row_w), dev(tq), dev(ts), I,
                                              kflags, offsets32=dev(off32), row_src=dev(row_src), R_max=R)
    else:
        hq, hs, hTq, hTs = moe.moe_grouped_w1(pw, counts_d, dev(offsets), dev(row_w), dev(xq), dev(xs), I,
                                              kflags, offsets32=dev(off32))
    dh = _h_error_bound(xq, xs, offsets, w1, fmt, I, ref, wts)
    assert_mx_within_1ulp(host(hq)[:R], host(hs)[:R], ref.hq, ref.hs, "h", extra_tol=dh)
    if transpose:
        q_ref, s_ref = omoe.concat_transposed(ref.hTq, ref.hTs, I)
        n = q_ref.shape[1]
        dhT = np.zeros((I, n))
        col = 0
        for g in range(G):
            lo, hi = offsets[g], offsets[g + 1]
            dhT[:, col:col + hi - lo] = dh[lo:hi].T
            col += (hi - lo + 31) // 32 * 32
        assert_mx_within_1ulp(host(hTq)[:, :n], host(hTs)[:, :n // 32], q_ref, s_ref, "hT",
                              extra_tol=dhT)


def _h_error_bound(xq, xs, offsets, w1, fmt, I, ref, wts):
    """Propagate the MFMA inner-sum bound (MFMA_REL * sum |x w|) on the gate
    and up sums through h = SiLU(g) * u * w; |SiLU'| <= 1.1."""
    X = np.abs(mx.dequantize_mx(xq, xs, mx.FMT_E4M3))
    mag = np.zeros_like(ref.acc)
    for g in range(len(offsets) - 1):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            mag[lo:hi] = X[lo:hi] @ np.abs(mx.dequantize_mx(w1[g][0], w1[g][1], fmt)).T
    dg, du = MFMA_REL * mag[:, :I], MFMA_REL * mag[:, I:]
    gate, up = ref.acc[:, :I], ref.acc[:, I:]
    return (1.1 * (np.abs(up) + du) * dg + np.abs(omoe.silu(gate)) * du) * np.abs(wts)[:, None]


W2_CASES = [
    ([0, 1, 17, 70, 33, 5], 1024, 512, "e2m1"),
    ([3, 0, 64, 129], 512, 256, "e4m3"),
    ([200], 768, 384, "e2m1"),
    ([0, 1, 255, 256, 257, 600, 33], 512, 256, "e4m3"),
    ([300, 17, 513], 1024, 512, "e2m1"),
    ([128, 384, 0, 129, 640, 1], 1024, 256, "e4m3"),
    # 9 groups x 64 units: four waves per workgroup, half units
    ([5, 1, 0, 20, 3, 7, 2, 16, 40], 4096, 256, "e4m3"),
    # 32 groups x 32 units: two waves per workgroup, half units
    ([(5 * g) % 9 + 1 for g in range(32)], 2048, 1024, "e2m1"),
    # 80 groups x 64 units: two waves per workgroup, whole units
    ([(3 * g) % 7 + 1 for g in range(80)], 4096, 256, "e4m3"),
    # 40 groups x 56 units: 2240 units on two-wave workgroups, half units
    # (2.2 rounds of halves against 2 of whole units)
    ([(3 * g) % 7 + 1 for g in range(40)], 3584, 512, "e2m1"),
    # 16 weight tiles (H = 4096) x about 50 row passes: three or four work
    # items per workgroup of the LDS-tiled kernel, ragged tails
    ([5000, 257, 0, 3100, 2555, 1031], 4096, 256, "e4m3"),
    ([4100, 6000, 1, 1955], 4096, 384, "e2m1"),
    # one K-tile (I = 128) and several items per workgroup: no weight tiles
    # requested ahead, every step an item's last
    ([5000, 257, 0, 3100, 2555, 1031], 4096, 128, "e2m1"),
    # a long K (I = 4096, 32 K-tiles): K-chunked staging with 64-row passes
    ([40, 90, 3, 0, 71], 512, 4096, "e2m1"),
]


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("counts,H,I,fmt", W2_CASES)
def test_grouped_w2_parity(counts, H, I, fmt, kernel):
    banner(f"grouped_w2 {kernel} counts={counts} H={H} I={I} fmt={fmt}")
    offsets, _, _, _, _, w2 = _grouped_problem(counts, H, I, fmt, 9 + H + I)
    R = int(offsets[-1])
    rng = np.random.default_rng(1)
    hq, hs = mx.quantize_mx(rng.standard_normal((R, I)) * 0.1, mx.FMT_E4M3)
    y_ref = omoe.grouped_w2(hq, hs, offsets, [a[0] for a in w2], [a[1] for a in w2], fmt)
    pw = _packed(w2, fmt, False)
    y = moe.moe_grouped_w2(pw, dev(np.array(counts, np.int32)), dev(offsets), dev(hq), dev(hs), H,
                           flags=KERNELS[kernel])
    # tolerance: one BF16 step, plus the scaled-MFMA inner-sum bound for
    # outputs that cancel
    hd = mx.dequantize_mx(hq, hs, mx.FMT_E4M3)
    mag = np.zeros((R, H))
    for g in range(len(counts)):
        lo, hi = offsets[g], offsets[g + 1]
        if hi > lo:
            W = mx.dequantize_mx(w2[g][0], w2[g][1], fmt)
            mag[lo:hi] = np.abs(hd[lo:hi]) @ np.abs(W).T
    assert_bf16_close(bf16_bits(y)[:R], y_ref, "y", max_ulp=1, abs_floor=MFMA_REL * mag, mag=mag)


# ------------------------------------------------------------------- combine
@pytest.mark.parametrize("T", [37, 1025])
@pytest.mark.parametrize("with_weight", [False, True])
def test_combine_bit_exact(with_weight, T):
    banner(f"combine with_weight={with_weight} T={T}")
    rng = np.random.default_rng(3)
    ks, H, R = 9, 1024, 200
    y = mx.bf16_rne(rng.standard_normal((R, H)) * 10.0 ** rng.uniform(-3, 3, (R, 1)))
    slot = rng.integers(-1, R, (T, ks)).astype(np.int32)
    slot[0] = -1                                          # token with no local slot
    row_w = rng.uniform(0, 1, R).astype(np.float32)
    ref = omoe.combine(y, slot, H, row_w.astype(np.float64) if with_weight else None)
    out = moe.moe_combine(dev(y.view(np.int16)).view(torch.uint16), dev(slot), H,
                          row_w=dev(row_w) if with_weight else None)
    np.testing.assert_array_equal(bf16_bits(out), ref)


# ------------------------------------------------------- HBM read-rate probe
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 1024 * 16 * 3])
def test_hbm_read_probe_reads_every_chunk(nbytes):
    """The probe's XOR of all sink words equals the XOR of every 4-byte word
    of the buffer, so every chunk was read once, including a ragged last
    pass."""
    banner(f"hbm read probe {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = dev(words.view(np.int32))
    sink = moe.moe_hbm_read_probe(src)
    got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
