"""Plain CPU definition of one GPU's share of a routed MoE layer, fp64.

Test infrastructure only (see the package header).

The steps and their order follow the GC-MoE summary page ("Approach": routing
counts, W1 on ready token blocks, an epilogue that fuses SwiGLU, routing-weight
scaling and FP8 requantisation, W2 producing BF16 fragments, then combine;
"Key contributions": the fused epilogue and optional shared expert) and the
fusion-kernel blog (SwiGLU definition in the "GLU activation in a fused GEMM
epilogue" section; per-group token counts kept in device memory in the
"Removing host-device synchronisation" section; the MXFP8 transposed copy in
the "Fusing MXFP8/NVFP4 quantisation" section).

Where the pages are silent the readings are:
* router: softmax over all experts' fp32 logits; the k largest logits are
  selected (ties to the lower expert id), in descending order; weights are the
  softmax probabilities, not renormalised unless asked;
* only experts [e0, e0 + n_local) are computed here; a token with no local
  slot contributes an exact zero row;
* grouping is stable: within an expert, rows follow the flattened assignment
  index t*k + j; experts in ascending local id; the shared expert (if any) is
  the last group and takes every token in order with weight 1;
* W1 rows [0, I) are the gate (through SiLU, beta = 1), rows [I, 2I) are up;
  no bias; the routing weight multiplies h once, before requantisation;
* quantisation points: h -> MX-E4M3 (blocks of 32 along I), y -> BF16 per
  row, out -> BF16; every other step is exact or fp64.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import mx


# ------------------------------------------------------------------ routing
def route(logits: np.ndarray, k: int, renorm: bool = False):
    """Top-k softmax router.

    logits: float32 [T, E].  Returns (topk_idx int32 [T, k], topk_w fp64 [T, k]).
    Selection compares the fp32 logits themselves (softmax is strictly
    increasing, so this selects the k largest probabilities) with ties going
    to the lower expert id; slot j holds the j-th largest.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    assert 1 <= k <= E
    assert np.all(np.isfinite(logits)), "router logits must be finite"
    ids = np.broadcast_to(np.arange(E), (T, E))
    # np.lexsort: last key is primary; it is stable, so equal logits keep id order.
    order = np.lexsort((ids, -logits.astype(np.float64)), axis=-1)
    topk_idx = order[:, :k].astype(np.int32)
    l64 = logits.astype(np.float64)
    m = l64.max(axis=1, keepdims=True)
    ex = np.exp(l64 - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    topk_w = np.take_along_axis(p, topk_idx.astype(np.int64), axis=1)
    if renorm:
        topk_w = topk_w / topk_w.sum(axis=1, keepdims=True)
    return topk_idx, topk_w


# --------------------------------------------------- counts and permutation
@dataclass
class Permutation:
    counts: np.ndarray      # int32 [G]
    offsets: np.ndarray     # int32 [G + 1], offsets[0] = 0
    row_src: np.ndarray     # int32 [R]   source token of each grouped row
    row_slot: np.ndarray    # int32 [R]   slot j of that token (k for the shared group)
    row_w: np.ndarray       # fp64  [R]   routing weight of each row
    slot_row: np.ndarray    # int32 [T, k + s], -1 where the slot is not local
    G: int = 0
    E_loc: int = 0
    shared: bool = False


def permute(topk_idx: np.ndarray, topk_w: np.ndarray, e0: int, n_local: int,
            shared: bool = False) -> Permutation:
    """Group the local assignments by expert, stably (see the module header)."""
    T, k = topk_idx.shape
    s = 1 if shared else 0
    G = n_local + s
    lists = [[] for _ in range(G)]
    for a in range(T * k):                      # flattened assignment index
        t, j = divmod(a, k)
        g = int(topk_idx[t, j]) - e0
        if 0 <= g < n_local:
            lists[g].append((t, j, float(topk_w[t, j])))
    if shared:
        lists[n_local] = [(t, k, 1.0) for t in range(T)]
    counts = np.array([len(lst) for lst in lists], dtype=np.int32)
    offsets = np.zeros(G + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    row_src = np.zeros(R, dtype=np.int32)
    row_slot = np.zeros(R, dtype=np.int32)
    row_w = np.zeros(R, dtype=np.float64)
    slot_row = np.full((T, k + s), -1, dtype=np.int32)
    for g, lst in enumerate(lists):
        for i, (t, j, w) in enumerate(lst):
            r = offsets[g] + i
            row_src[r], row_slot[r], row_w[r] = t, j, w
            slot_row[t, j] = r
    return Permutation(counts, offsets, row_src, row_slot, row_w, slot_row, G, n_local, shared)


def gather_rows(xq: np.ndarray, xs: np.ndarray, perm: Permutation):
    """Copy each grouped row's FP8 codes and E8M0 scales from its source token."""
    return xq[perm.row_src], xs[perm.row_src]


# -------------------------------------------------------------- expert MLP
def silu(g: np.ndarray) -> np.ndarray:
    """Swish with beta = 1: g * sigmoid(g), fp64."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_rows(acc: np.ndarray, I: int, w: np.ndarray) -> np.ndarray:
    """h = SiLU(gate) * up * w for W1 output rows acc [n, 2I] (gate first)."""
    gate, up = acc[:, :I], acc[:, I:2 * I]
    return silu(gate) * up * np.asarray(w, dtype=np.float64)[:, None]


# ------------------------------------------- epilogue variants and backward
# The fusion blog's GLU section writes the gated unit as
# SwiGLU(x, W, V, b, c, beta) = Swish_beta(xW + b) (x) (xV + c) and names GeGLU
# and sReLU as the other supported activations, with clamping and bias
# addition as fused options; its kernel list has a backward member,
# "GroupGemm + dActivation + Quantize/Transpose", whose epilogue reads the
# GEMM output, forms the activation's derivative and quantises it. Readings
# (the page gives no further definition):
#  * every variant keeps the two-chunk structure: rows [0, I) of W1 feed the
#    activation (the gate), rows [I, 2I) multiply it (up);
#  * GeGLU uses the exact GELU, z * Phi(z) with the normal CDF Phi;
#  * sReLU is the squared ReLU max(z, 0)^2 applied to the gate chunk;
#  * the bias (b for the gate, c for up) is added to the GEMM output, then
#    the clamp limits both chunks to [-limit, limit] (limit 0: no clamp);
#  * beta is Swish's slope (SwiGLU only; beta = 1 is SiLU).
ACT_SWIGLU, ACT_GEGLU, ACT_SRELU = 0, 1, 2


def _normal_cdf(z):
    from math import erf
    return 0.5 * (1.0 + np.vectorize(erf, otypes=[np.float64])(z / np.sqrt(2.0)))


def _normal_pdf(z):
    return np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


def activation(z, act: int = ACT_SWIGLU, beta: float = 1.0):
    """The gate activation a(z), fp64."""
    z = np.asarray(z, dtype=np.float64)
    if act == ACT_SWIGLU:
        with np.errstate(over="ignore"):
            return z / (1.0 + np.exp(-beta * z))
    if act == ACT_GEGLU:
        return z * _normal_cdf(z)
    if act == ACT_SRELU:
        return np.maximum(z, 0.0) ** 2
    raise ValueError(act)


def activation_grad(z, act: int = ACT_SWIGLU, beta: float = 1.0):
    """da/dz, fp64: Swish_beta: s + beta z s (1 - s) with s = sigmoid(beta z);
    GELU: Phi(z) + z phi(z); squared ReLU: 2 max(z, 0)."""
    z = np.asarray(z, dtype=np.float64)
    if act == ACT_SWIGLU:
        with np.errstate(over="ignore"):
            sg = 1.0 / (1.0 + np.exp(-beta * z))
        return sg + beta * z * sg * (1.0 - sg)
    if act == ACT_GEGLU:
        return _normal_cdf(z) + z * _normal_pdf(z)
    if act == ACT_SRELU:
        return 2.0 * np.maximum(z, 0.0)
    raise ValueError(act)


def preactivation(acc, I: int, bias=None, limit: float = 0.0):
    """Gate and up chunks after the bias and the clamp: (g, u), each [n, I]."""
    acc = np.asarray(acc, dtype=np.float64)
    g, u = acc[:, :I], acc[:, I:2 * I]
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)
        g, u = g + b[:I], u + b[I:2 * I]
    if limit > 0:
        g, u = np.clip(g, -limit, limit), np.clip(u, -limit, limit)
    return g, u


def glu_rows(acc, I: int, w, act: int = ACT_SWIGLU, beta: float = 1.0, bias=None,
             limit: float = 0.0):
    """h = a(g) * u * w for W1 output rows acc [n, 2I] (gate first), with the
    bias, clamp and activation of the variant; SwiGLU with beta = 1 and no
    bias or clamp is swiglu_rows."""
    g, u = preactivation(acc, I, bias, limit)
    return activation(g, act, beta) * u * np.asarray(w, dtype=np.float64)[:, None]


def glu_backward_rows(pre, dh, I: int, w, act: int = ACT_SWIGLU, beta: float = 1.0,
                      limit: float = 0.0):
    """Backward of h = a(clamp(g)) * clamp(u) * w for rows of the saved
    pre-activation pre = [g | u] ([n, 2I], bias included, before the clamp)
    and the incoming gradient dh [n, I]:
      dg = dh * w * clamp(u) * a'(clamp(g)) * [|g| <= limit]
      du = dh * w * a(clamp(g)) * [|u| <= limit]
      dw = sum_i dh * a(clamp(g)) * clamp(u)
    (the clamp passes the gradient where |z| <= limit; without a clamp the
    masks are 1). Returns (d_pre [n, 2I], dw [n])."""
    pre = np.asarray(pre, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)[:, None]
    g, u = pre[:, :I], pre[:, I:2 * I]
    mg = np.ones_like(g) if limit <= 0 else (np.abs(g) <= limit).astype(np.float64)
    mu = np.ones_like(u) if limit <= 0 else (np.abs(u) <= limit).astype(np.float64)
    gc = g if limit <= 0 else np.clip(g, -limit, limit)
    uc = u if limit <= 0 else np.clip(u, -limit, limit)
    a = activation(gc, act, beta)
    dg = dh * w * uc * activation_grad(gc, act, beta) * mg
    du = dh * w * a * mu
    dw = np.sum(dh * a * uc, axis=1)
    return np.concatenate([dg, du], axis=1), dw


@dataclass
class BwdOut:
    dq: np.ndarray                          # uint8 [R, 2I]   E4M3 codes of [dg | du]
    ds: np.ndarray                          # uint8 [R, 2I/32]
    d: np.ndarray                           # fp64  [R, 2I]   unrounded
    dh: np.ndarray                          # fp64  [R, I]    the GEMM output
    dw: np.ndarray                          # fp64  [R]
    dTq: list = field(default_factory=list)   # per group uint8 [2I, roundup(n_g, 32)]
    dTs: list = field(default_factory=list)


def grouped_w1_backward(dq_tok, ds_tok, row_src, offsets, row_w, pre_bits, w2tq, w2ts,
                        w_fmt: str, I: int, act: int = ACT_SWIGLU, beta: float = 1.0,
                        limit: float = 0.0, transpose: bool = False, rule: str = "ocp",
                        groups=None) -> BwdOut:
    """The backward GEMM of the fused W1 epilogue, per group g:
      dh = dec(dout rows) @ dec(W2T_g)^T      (fp64; W2T_g = W2_g^T [I, H],
                                              MX-quantised along H)
      [dg | du], dw = glu_backward_rows(bf16 pre-activation rows, dh, ...)
    then [dg | du] requantised to MX-E4M3 along the 2I features and, with
    `transpose`, per group in blocks of 32 rows (as the forward's transposed
    copy). dq_tok/ds_tok: the gradient of the layer output, E4M3 codes
    [T, H] and E8M0 scales [T, H/32]; grouped row r reads token row_src[r].
    pre_bits: bf16 bits [R, 2I] of the saved pre-activation."""
    R = int(offsets[-1])
    G = len(offsets) - 1
    dh = np.zeros((R, I))
    d = np.zeros((R, 2 * I))
    dw = np.zeros(R)
    todo = range(G) if groups is None else groups
    pre = mx.bf16_value(np.asarray(pre_bits))
    for g in todo:
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            src = np.asarray(row_src[lo:hi])
            D = mx.dequantize_mx(np.asarray(dq_tok)[src], np.asarray(ds_tok)[src], mx.FMT_E4M3)
            W = mx.dequantize_mx(np.asarray(w2tq[g]), np.asarray(w2ts[g]), w_fmt)
            dh[lo:hi] = D @ W.T
            d[lo:hi], dw[lo:hi] = glu_backward_rows(pre[lo:hi], dh[lo:hi], I, row_w[lo:hi], act,
                                                     beta, limit)
    q, sc = mx.quantize_mx(d, mx.FMT_E4M3, rule)
    out = BwdOut(q, sc, d, dh, dw)
    if transpose:
        for g in range(G):
            lo, hi = int(offsets[g]), int(offsets[g + 1])
            tq, ts = quantize_transposed(d[lo:hi], rule)
            out.dTq.append(tq)
            out.dTs.append(ts)
    return out


def quantize_transposed(h: np.ndarray, rule: str = "ocp"):
    """Transposed MX-E4M3 copy of one expert's h [n, I]: hT [I, n32] with
    n32 = roundup(n, 32), quantised in blocks of 32 tokens counted from the
    expert's first row. A partial last block takes its amax over the valid
    tokens only; its padding columns hold code 0."""
    n, I = h.shape
    n32 = -(-n // 32) * 32
    hT = np.zeros((I, n32), dtype=np.float64)
    hT[:, :n] = h.T
    q, sc = mx.quantize_mx(hT, mx.FMT_E4M3, rule)
    q[:, n:] = 0
    return q, sc


@dataclass
class W1Out:
    hq: np.ndarray                       # uint8 [R, I]
    hs: np.ndarray                       # uint8 [R, I/32]
    h: np.ndarray                        # fp64  [R, I]   unrounded
    acc: np.ndarray                      # fp64  [R, 2I]
    hTq: list = field(default_factory=list)   # per group uint8 [I, roundup(n_g,32)]
    hTs: list = field(default_factory=list)   # per group uint8 [I, roundup(n_g,32)/32]


def grouped_w1(xq_perm, xs_perm, offsets, row_w, w1q, w1s, w1_fmt: str, I: int,
               transpose: bool = False, rule: str = "ocp", groups=None, act: int = ACT_SWIGLU,
               beta: float = 1.0, bias=None, limit: float = 0.0) -> W1Out:
    """Per group g: acc = X_g @ W1_g^T in fp64, then the fused epilogue.

    xq_perm/xs_perm: E4M3 codes [R, H] and E8M0 scales [R, H/32].
    w1q/w1s: per-group sequences of W1 codes [2I, H(*1/2 for FP4)] and scales [2I, H/32].
    `groups` optionally restricts the computation to a subset of group ids.
    act/beta/bias/limit: the epilogue variant (see glu_rows); bias is per
    group [G][2I] or None. The default is SwiGLU with beta = 1.
    """
    R = int(offsets[-1])
    G = len(offsets) - 1
    acc = np.zeros((R, 2 * I))
    h = np.zeros((R, I))
    hTq, hTs = [], []
    todo = range(G) if groups is None else groups
    for g in todo:
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            X = mx.dequantize_mx(xq_perm[lo:hi], xs_perm[lo:hi], mx.FMT_E4M3)
            W = mx.dequantize_mx(np.asarray(w1q[g]), np.asarray(w1s[g]), w1_fmt)
            acc[lo:hi] = X @ W.T
            if act == ACT_SWIGLU and beta == 1.0 and bias is None and limit <= 0:
                h[lo:hi] = swiglu_rows(acc[lo:hi], I, row_w[lo:hi])
            else:
                h[lo:hi] = glu_rows(acc[lo:hi], I, row_w[lo:hi], act, beta,
                                    None if bias is None else bias[g], limit)
    hq, hs = mx.quantize_mx(h, mx.FMT_E4M3, rule)
    if transpose:
        for g in range(G):
            lo, hi = int(offsets[g]), int(offsets[g + 1])
            q, sc = quantize_transposed(h[lo:hi], rule)
            hTq.append(q)
            hTs.append(sc)
    return W1Out(hq, hs, h, acc, hTq, hTs)


def concat_transposed(hTq_list, hTs_list, I: int):
    """Lay the per-group transposed copies side by side: [I, sum roundup(n_g,32)]."""
    q = np.concatenate([np.asarray(x).reshape(I, -1) for x in hTq_list], axis=1) \
        if hTq_list else np.zeros((I, 0), np.uint8)
    s = np.concatenate([np.asarray(x).reshape(I, -1) for x in hTs_list], axis=1) \
        if hTs_list else np.zeros((I, 0), np.uint8)
    return q, s


def grouped_w2(hq, hs, offsets, w2q, w2s, w2_fmt: str, groups=None, H: int | None = None):
    """Per group g: y_g = BF16_RNE(dec(h_g) @ dec(W2_g)^T), rounded once from fp64.
    Groups with no rows are never read (their entries may be None); H defaults
    to the row count of the first group's W2."""
    R = int(offsets[-1])
    G = len(offsets) - 1
    if H is None:
        H = next(np.asarray(s).shape[0] for s in w2s if s is not None)
    yv = np.zeros((R, H))
    todo = range(G) if groups is None else groups
    for g in todo:
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            Hd = mx.dequantize_mx(hq[lo:hi], hs[lo:hi], mx.FMT_E4M3)
            W = mx.dequantize_mx(np.asarray(w2q[g]), np.asarray(w2s[g]), w2_fmt)
            yv[lo:hi] = Hd @ W.T
    return mx.bf16_rne(yv)


def combine(y_bits: np.ndarray, slot_row: np.ndarray, H: int, row_scale=None):
    """out[t] = BF16_RNE(sum over the token's local slots of y rows), summed in
    fp64; a token with no local slot gives +0. `row_scale` (optional, per grouped
    row) multiplies each row first: the weight-at-combine variant."""
    T = slot_row.shape[0]
    acc = np.zeros((T, H))
    yv = mx.bf16_value(y_bits)
    for t in range(T):
        for r in slot_row[t]:
            if r >= 0:
                acc[t] += yv[r] if row_scale is None else yv[r] * row_scale[r]
    return mx.bf16_rne(acc)


# ---------------------------------------------------------------- the layer
@dataclass
class LayerOut:
    out: np.ndarray          # uint16 bf16 [T, H]
    topk_idx: np.ndarray
    topk_w: np.ndarray
    perm: Permutation
    w1: W1Out
    y: np.ndarray            # uint16 bf16 [R, H]


def moe_layer(logits, xq, xs, k: int, w1q, w1s, w2q, w2s, w_fmt: str, I: int,
              e0: int = 0, n_local: int | None = None, shared=None,
              renorm: bool = False, transpose: bool = False,
              weight_at_combine: bool = False, rule: str = "ocp", epi=None) -> LayerOut:
    """One GPU's share of the routed MoE layer, from quantised inputs to BF16.

    logits f32 [T, E_tot]; xq uint8 E4M3 [T, H]; xs uint8 E8M0 [T, H/32];
    w1q/w1s/w2q/w2s: per local expert codes and scales (see grouped_w1/w2);
    shared: None or (sw1q, sw1s, sw2q, sw2s) for an always-on shared expert.
    epi: None (SwiGLU) or a dict of the epilogue variant: act, beta, limit and
    bias (per group [G][2I], the shared expert's last, or None).
    """
    E_tot = logits.shape[1]
    n_local = E_tot if n_local is None else n_local
    idx, w = route(logits, k, renorm)
    perm = permute(idx, w, e0, n_local, shared is not None)
    xq_p, xs_p = gather_rows(np.asarray(xq), np.asarray(xs), perm)
    w1q_g, w1s_g, w2q_g, w2s_g = list(w1q), list(w1s), list(w2q), list(w2s)
    if shared is not None:
        w1q_g.append(shared[0]); w1s_g.append(shared[1])
        w2q_g.append(shared[2]); w2s_g.append(shared[3])
    row_w_h = np.ones_like(perm.row_w) if weight_at_combine else perm.row_w
    o1 = grouped_w1(xq_p, xs_p, perm.offsets, row_w_h, w1q_g, w1s_g, w_fmt, I,
                    transpose=transpose, rule=rule, **(epi or {}))
    H = xq.shape[1]
    y = grouped_w2(o1.hq, o1.hs, perm.offsets, w2q_g, w2s_g, w_fmt, H=H)
    out = combine(y, perm.slot_row, H, perm.row_w if weight_at_combine else None)
    return LayerOut(out, idx, w, perm, o1, y)


def expert_output(x_row: np.ndarray, w1q, w1s, w2q, w2s, w_fmt: str, I: int, weight: float,
                  rule: str = "ocp", epi=None, bias=None) -> np.ndarray:
    """One expert's contribution for one token, from dequantised x [H]:
    BF16 value of W2 . Q8(SiLU(gate) * up * weight), fp64 inside (or the
    epilogue variant `epi`, with this expert's `bias`)."""
    acc = x_row[None, :] @ mx.dequantize_mx(np.asarray(w1q), np.asarray(w1s), w_fmt).T
    if epi is None:
        h = swiglu_rows(acc, I, np.array([weight]))
    else:
        h = glu_rows(acc, I, np.array([weight]), epi.get("act", ACT_SWIGLU), epi.get("beta", 1.0),
                     bias, epi.get("limit", 0.0))
    hq, hs = mx.quantize_mx(h, mx.FMT_E4M3, rule)
    yv = mx.dequantize_mx(hq, hs, mx.FMT_E4M3) @ \
        mx.dequantize_mx(np.asarray(w2q), np.asarray(w2s), w_fmt).T
    return mx.bf16_value(mx.bf16_rne(yv))[0]


def token_output(logit_row, xq_row, xs_row, k: int, get_expert, w_fmt: str, I: int,
                 e0: int = 0, n_local: int | None = None, shared=None, rule: str = "ocp",
                 weight_at_combine: bool = False, epi=None):
    """Brute-force output of one token: route it, run each local slot's expert
    MLP on it alone, sum in fp64, round to BF16. `get_expert(g)` returns the
    local expert's (w1q, w1s, w2q, w2s) codes, so weights can be produced on
    demand; `shared` is the shared expert's codes or None. With
    weight_at_combine the routing weight is not applied inside the expert
    (h is quantised unweighted) but to the expert's BF16 output, in fp64,
    when the slots are summed. Returns bf16 bits [H]."""
    logit_row = np.asarray(logit_row, dtype=np.float32)[None, :]
    E_tot = logit_row.shape[1]
    n_local = E_tot if n_local is None else n_local
    idx, w = route(logit_row, k)
    x = mx.dequantize_mx(np.asarray(xq_row)[None, :], np.asarray(xs_row)[None, :], mx.FMT_E4M3)[0]
    out = np.zeros(x.shape[0])
    bias = (epi or {}).get("bias")
    for j in range(k):
        g = int(idx[0, j]) - e0
        if 0 <= g < n_local:
            wj = float(w[0, j])
            b = None if bias is None else bias[g]
            if weight_at_combine:
                out += expert_output(x, *get_expert(g), w_fmt, I, 1.0, rule, epi, b) * wj
            else:
                out += expert_output(x, *get_expert(g), w_fmt, I, wj, rule, epi, b)
    if shared is not None:
        out += expert_output(x, *shared, w_fmt, I, 1.0, rule, epi, None if bias is None else bias[n_local])
    return mx.bf16_rne(out)


def dense_layer(logits, xq, xs, k: int, w1q, w1s, w2q, w2s, w_fmt: str, I: int,
                e0: int = 0, n_local: int | None = None, shared=None, rule: str = "ocp",
                weight_at_combine: bool = False, epi=None):
    """Brute-force evaluation with no grouping: every token on its own (see
    token_output). Returns bf16 bits [T, H]. Used to pin the grouped computation."""
    T = logits.shape[0]
    get = lambda g: (w1q[g], w1s[g], w2q[g], w2s[g])  # noqa: E731
    rows = [token_output(logits[t], xq[t], xs[t], k, get, w_fmt, I, e0, n_local, shared, rule,
                         weight_at_combine, epi)
            for t in range(T)]
    return np.stack(rows) if rows else np.zeros((0, xq.shape[1]), np.uint16)


# ------------------------------------------------------- algorithmic work
def algorithmic_bytes(T: int, E_tot: int, H: int, I: int, active_groups: int,
                      w_fmt: str) -> int:
    """HBM bytes the method must move per call: logits, x (codes + scales), the
    W1 + W2 codes and scales of the active groups only, and the BF16 output."""
    bw = 0.5 if w_fmt == mx.FMT_E2M1 else 1.0
    per_group = int(3 * I * H * bw) + 3 * I * H // 32
    return 4 * T * E_tot + T * H + T * H // 32 + active_groups * per_group + 2 * T * H


def algorithmic_flops(R: int, H: int, I: int) -> int:
    """Multiply-add work of the two grouped GEMMs over real rows: 6 R H I."""
    return 6 * R * H * I
