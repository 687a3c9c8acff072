"""routed_grouped_gemm_amd: one GPU's share of a routed MoE layer on MI355X.

A thin PyTorch binding over libmoe (include/moe.h). Every function here only
marshals arguments (device pointers, sizes, the current HIP stream) and calls
the C ABI of the same name; all computation runs in the library's HIP kernels.
PyTorch provides device memory and streams. Importing the package fails if the
library has not been built (python routed_grouped_gemm_amd/build.py).
"""
from __future__ import annotations

import contextlib
import ctypes as C

import torch

from . import _lib
from ._lib import (MOE_ACT_GEGLU, MOE_ACT_SRELU, MOE_ACT_SWIGLU, MOE_FMT_MXFP4,  # noqa: F401
                   MOE_FMT_MXFP8, MOE_GEMM_PASS, MOE_GEMM_STREAMED, MOE_GEMM_TILED,
                   MOE_LAYER_SEPARATE_KERNELS,
                   MOE_LAYER_TOKEN_RING, MOE_ROUTE_RENORM,
                   MOE_SCALE_RULE_CEIL, MOE_W1_WRITE_TRANSPOSE, MOE_WEIGHT_AT_COMBINE,
                   moe_epilogue, moe_layer_args, moe_weights)

lib = _lib.load()


class MoeError(RuntimeError):
    pass


def _check(status: int, name: str) -> None:
    if status != 0:
        raise MoeError(f"{name} failed: {lib.moe_status_string(status).decode()} (status {status})")


def _p(t):
    return None if t is None else t.data_ptr()


def _on(stream):
    """Context in which a wrapper allocates and launches: `stream` made the
    current stream (so the caching allocator ties every temporary and output
    to the stream whose kernels use it), or the current stream left as it is."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _stream():
    """Handle of the current stream (inside `_on`, the caller's stream)."""
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if t.device.type != "cuda":
        raise MoeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    return t


def version() -> str:
    return lib.moe_version().decode()


# ------------------------------------------------------------------ weights
def moe_prepacked_size(G: int, N: int, K: int, fmt: int) -> int:
    return int(lib.moe_prepacked_size(G, N, K, fmt))


def moe_quantize_mx(src: torch.Tensor, fmt: int, flags: int = 0, q=None, s=None, stream=None):
    """fp32 [rows, K] -> (codes, E8M0 scales); codes are [rows, K] E4M3 or
    [rows, K/2] packed E2M1."""
    _dev(src, torch.float32, "src")
    rows, K = src.shape
    with _on(stream):
        if q is None:
            q = torch.empty((rows, K if fmt == MOE_FMT_MXFP8 else K // 2), dtype=torch.uint8,
                            device=src.device)
        if s is None:
            s = torch.empty((rows, K // 32), dtype=torch.uint8, device=src.device)
        _check(lib.moe_quantize_mx(_p(src), rows, K, fmt, flags, _p(q), _p(s), _stream()),
               "moe_quantize_mx")
    return q, s


MOE_HBM_PROBE_SINK_WORDS = 8192


def moe_hbm_read_probe(src: torch.Tensor, sink=None, stream=None):
    """One streaming read of the bytes of `src` (a measurement utility).
    Returns sink (uint32 words, int32 dtype); their XOR is the XOR of the
    buffer's 4-byte words."""
    if not src.is_cuda or not src.is_contiguous():
        raise MoeError("src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    with _on(stream):
        if sink is None:
            sink = torch.empty(MOE_HBM_PROBE_SINK_WORDS, dtype=torch.int32, device=src.device)
        _check(lib.moe_hbm_read_probe(_p(src), nbytes, _p(sink), _stream()), "moe_hbm_read_probe")
    return sink


class PackedWeights:
    """Prepacked expert weights (device buffer + its moe_weights descriptor)."""

    def __init__(self, q: torch.Tensor, s: torch.Tensor, fmt: int, is_w1: bool, stream=None):
        _dev(q, torch.uint8, "q")
        _dev(s, torch.uint8, "s")
        G, N = q.shape[0], q.shape[1]
        K = s.shape[2] * 32
        nbytes = moe_prepacked_size(G, N, K, fmt)
        if nbytes == 0:
            raise MoeError(f"bad weight shape G={G} N={N} K={K}")
        with _on(stream):
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
            _check(lib.moe_prepack_weights(_p(q), _p(s), G, N, K, fmt, int(is_w1), _p(self.buf),
                                           nbytes, _stream()), "moe_prepack_weights")
        self.desc = moe_weights(fmt, G, N, K, int(is_w1), 0, _p(self.buf), nbytes)
        self.G, self.N, self.K, self.fmt, self.is_w1 = G, N, K, fmt, bool(is_w1)

    @classmethod
    def empty(cls, G: int, N: int, K: int, fmt: int, is_w1: bool, device="cuda"):
        """An unfilled buffer of the right size (filled later, e.g. one group at a time)."""
        self = cls.__new__(cls)
        nbytes = moe_prepacked_size(G, N, K, fmt)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.desc = moe_weights(fmt, G, N, K, int(is_w1), 0, _p(self.buf), nbytes)
        self.G, self.N, self.K, self.fmt, self.is_w1 = G, N, K, fmt, bool(is_w1)
        return self

    @property
    def group_stride(self) -> int:
        return moe_prepacked_size(1, self.N, self.K, self.fmt)

    def fill_group(self, g: int, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
        """Prepack one expert's logical codes q [N, K or K/2] and scales s [N, K/32]
        into group slot g."""
        _dev(q, torch.uint8, "q")
        _dev(s, torch.uint8, "s")
        st = self.group_stride
        dst = self.buf[g * st:(g + 1) * st]
        with _on(stream):
            _check(lib.moe_prepack_weights(_p(q), _p(s), 1, self.N, self.K, self.fmt, int(self.is_w1),
                                           _p(dst), st, _stream()), "moe_prepack_weights")

    def ref(self):
        return C.byref(self.desc)


def _wref(w):
    return None if w is None else w.ref()


class Epilogue:
    """The W1 epilogue variant (moe_epilogue): activation (MOE_ACT_*), Swish
    slope beta, clamp limit (0: none), optional per-group bias f32 [G, 2I] and
    optional BF16 pre-activation output [R_max, 2I] (both device tensors,
    referenced here so they outlive the call)."""

    def __init__(self, act: int = MOE_ACT_SWIGLU, beta: float = 1.0, limit: float = 0.0, bias=None,
                 save_pre=None):
        if bias is not None:
            _dev(bias, torch.float32, "bias")
        if save_pre is not None:
            _dev(save_pre, torch.uint16, "save_pre")
        self.bias, self.save_pre = bias, save_pre
        self.desc = moe_epilogue(act, beta, limit, 0, _p(bias), _p(save_pre))

    def ref(self):
        return C.byref(self.desc)


def _eref(e):
    return None if e is None else e.ref()


# ------------------------------------------------------------------- route
def moe_route(logits: torch.Tensor, k: int, flags: int = 0, topk_idx=None, topk_w=None, stream=None):
    _dev(logits, torch.float32, "logits")
    T, E = logits.shape
    with _on(stream):
        if topk_idx is None:
            topk_idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
        if topk_w is None:
            topk_w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
        _check(lib.moe_route(_p(logits), T, E, k, flags, _p(topk_idx), _p(topk_w), _stream()),
               "moe_route")
    return topk_idx, topk_w


# ----------------------------------------------------------------- permute
def moe_permute(topk_idx, topk_w, e0: int, n_local: int, shared: bool, xq=None, xs=None,
                stream=None):
    """Returns a dict: counts, offsets, offsets32, row_src, row_w, slot_row,
    xq_perm, xs_perm (the last two only when xq/xs are given)."""
    _dev(topk_idx, torch.int32, "topk_idx")
    _dev(topk_w, torch.float32, "topk_w")
    T, k = topk_idx.shape
    s = int(bool(shared))
    G = n_local + s
    R_max = T * k + s * T
    dev = topk_idx.device
    H = xq.shape[1] if xq is not None else 256
    with _on(stream):
        out = dict(
            counts=torch.empty(G, dtype=torch.int32, device=dev),
            offsets=torch.empty(G + 1, dtype=torch.int32, device=dev),
            offsets32=torch.empty(G + 1, dtype=torch.int32, device=dev),
            row_src=torch.empty(max(R_max, 1), dtype=torch.int32, device=dev),
            row_w=torch.empty(max(R_max, 1), dtype=torch.float32, device=dev),
            slot_row=torch.empty((T, k + s), dtype=torch.int32, device=dev),
        )
        if xq is not None:
            _dev(xq, torch.uint8, "xq")
            _dev(xs, torch.uint8, "xs")
            out["xq_perm"] = torch.empty((max(R_max, 1), H), dtype=torch.uint8, device=dev)
            out["xs_perm"] = torch.empty((max(R_max, 1), H // 32), dtype=torch.uint8, device=dev)
        nws = int(lib.moe_permute_workspace_size(T, k, G))
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        _check(lib.moe_permute(_p(topk_idx), _p(topk_w), T, k, e0, n_local, s, _p(xq), _p(xs), H,
                               _p(out["counts"]), _p(out["offsets"]), _p(out["offsets32"]),
                               _p(out["row_src"]), _p(out["row_w"]), _p(out["slot_row"]),
                               _p(out.get("xq_perm")), _p(out.get("xs_perm")), _p(ws), nws,
                               _stream()), "moe_permute")
    return out


# ----------------------------------------------------------------- grouped
def moe_transposed_ld(R_max: int, G: int) -> int:
    return int(lib.moe_transposed_ld(R_max, G))


def moe_grouped_w1(w1: PackedWeights, counts, offsets, row_w, xq, xs, I: int,
                   flags: int = 0, w1_shared: PackedWeights | None = None, offsets32=None,
                   hq=None, hs=None, hTq=None, hTs=None, row_src=None,
                   R_max: int | None = None, epi: Epilogue | None = None, stream=None):
    """xq/xs: the grouped rows [R_max, H] (row_src None) or the token rows
    [T, H] read through row_src (then R_max must be given). The launch
    configuration follows R_max / counts.shape[0] (see include/moe.h)."""
    H = xq.shape[1]
    if R_max is None:
        R_max = xq.shape[0]
    G = counts.shape[0]
    dev = xq.device
    with _on(stream):
        if hq is None:
            hq = torch.empty((R_max, I), dtype=torch.uint8, device=dev)
        if hs is None:
            hs = torch.empty((R_max, I // 32), dtype=torch.uint8, device=dev)
        if (flags & MOE_W1_WRITE_TRANSPOSE) and hTq is None:
            ld = moe_transposed_ld(R_max, G)
            hTq = torch.empty((I, ld), dtype=torch.uint8, device=dev)
            hTs = torch.empty((I, ld // 32), dtype=torch.uint8, device=dev)
        nws = int(lib.moe_grouped_workspace_size(R_max, G, 2 * I, H))
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        _check(lib.moe_grouped_w1(w1.ref(), _wref(w1_shared), _p(counts), _p(offsets), _p(offsets32),
                                  _p(row_w), _p(xq), _p(xs), _p(row_src), xq.shape[0], R_max, H, I, G,
                                  _eref(epi), flags, _p(hq), _p(hs), _p(hTq), _p(hTs), _p(ws), nws,
                                  _stream()),
               "moe_grouped_w1")
    return hq, hs, hTq, hTs


def moe_grouped_w1_backward(w2t: PackedWeights, counts, offsets, row_w, dyq, dys, row_src, pre, I: int,
                            epi: Epilogue | None = None, flags: int = 0, offsets32=None,
                            w2t_shared: PackedWeights | None = None, want_dw: bool = True, stream=None):
    """The backward of the fused W1 epilogue: w2t holds W2^T per group (N = I,
    K = H), dyq/dys the layer output's gradient in token order [T, H] (E4M3 +
    E8M0), row_src the grouped rows' tokens, pre the saved BF16 pre-activation
    [R_max, 2I]. Returns a dict: dq [R_max, 2I], ds [R_max, 2I/32], dTq/dTs
    (with MOE_W1_WRITE_TRANSPOSE), dw [R_max] (with row_w and want_dw)."""
    R_max = pre.shape[0]
    H = dyq.shape[1]
    G = counts.shape[0]
    dev = dyq.device
    with _on(stream):
        out = dict(dq=torch.empty((R_max, 2 * I), dtype=torch.uint8, device=dev),
                   ds=torch.empty((R_max, 2 * I // 32), dtype=torch.uint8, device=dev),
                   dTq=None, dTs=None, dw=None)
        if flags & MOE_W1_WRITE_TRANSPOSE:
            ld = moe_transposed_ld(R_max, G)
            out["dTq"] = torch.zeros((2 * I, ld), dtype=torch.uint8, device=dev)
            out["dTs"] = torch.zeros((2 * I, ld // 32), dtype=torch.uint8, device=dev)
        if want_dw and row_w is not None:
            out["dw"] = torch.empty(R_max, dtype=torch.float32, device=dev)
        nws = int(lib.moe_backward_workspace_size(R_max, G, H, I))
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        _check(lib.moe_grouped_w1_backward(
            w2t.ref(), _wref(w2t_shared), _p(counts), _p(offsets), _p(offsets32), _p(row_w), _p(dyq),
            _p(dys), _p(row_src), dyq.shape[0], _p(pre), R_max, H, I, G, _eref(epi), flags,
            _p(out["dq"]), _p(out["ds"]), _p(out["dTq"]), _p(out["dTs"]), _p(out["dw"]), _p(ws), nws,
            _stream()), "moe_grouped_w1_backward")
    return out


def moe_grouped_w2(w2: PackedWeights, counts, offsets, hq, hs, H: int,
                   w2_shared: PackedWeights | None = None, y=None, flags: int = 0, stream=None):
    R_max, I = hq.shape
    G = counts.shape[0]
    with _on(stream):
        if y is None:
            y = torch.empty((R_max, H), dtype=torch.uint16, device=hq.device)
        nws = int(lib.moe_grouped_workspace_size(R_max, G, H, I))
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=hq.device)
        _check(lib.moe_grouped_w2(w2.ref(), _wref(w2_shared), _p(counts), _p(offsets), _p(hq), _p(hs),
                                  R_max, H, I, G, flags, _p(y), _p(ws), nws, _stream()),
               "moe_grouped_w2")
    return y


# ----------------------------------------------------------------- combine
def moe_combine(y, slot_row, H: int, row_w=None, out=None, stream=None):
    T, ks = slot_row.shape
    with _on(stream):
        if out is None:
            out = torch.empty((T, H), dtype=torch.uint16, device=y.device)
        _check(lib.moe_combine(_p(y), _p(slot_row), _p(row_w), T, ks, H, _p(out), _stream()),
               "moe_combine")
    return out


# ------------------------------------------------------------------- layer
_NAMES = ["topk_idx", "topk_w", "counts", "offsets", "offsets32", "row_src", "row_w", "slot_row",
          "hq", "hs", "y", "scratch", "ctrl"]


class LayerWorkspace:
    """Device workspace of moe_layer plus views of its intermediates."""

    def __init__(self, T, E_tot, k, E_loc, H, I, shared=False, flags=0, device="cuda"):
        s = int(bool(shared))
        self.shape = (T, E_tot, k, E_loc, H, I, s, flags)
        self.nbytes = int(lib.moe_layer_workspace_size(T, E_tot, k, E_loc, H, I, s, flags))
        self.buf = torch.empty(max(self.nbytes, 1), dtype=torch.uint8, device=device)
        offs = (C.c_size_t * len(_NAMES))()
        lib.moe_layer_workspace_offsets(T, E_tot, k, E_loc, H, I, s, flags, offs)
        self.offsets = list(offs)
        self.scratch_offset = self.offsets[_NAMES.index("scratch")]

    def view(self, name: str) -> torch.Tensor:
        T, E_tot, k, E_loc, H, I, s, _ = self.shape
        R = T * k + s * T
        G = E_loc + s
        shapes = {
            "topk_idx": ((T, k), torch.int32), "topk_w": ((T, k), torch.float32),
            "counts": ((G,), torch.int32), "offsets": ((G + 1,), torch.int32),
            "offsets32": ((G + 1,), torch.int32), "row_src": ((R,), torch.int32),
            "row_w": ((R,), torch.float32), "slot_row": ((T, k + s), torch.int32),
            "hq": ((R, I), torch.uint8), "hs": ((R, I // 32), torch.uint8),
            "y": ((R, H), torch.uint16),
            "ctrl": ((8 + G + H // 64,), torch.int32),
        }
        shp, dt = shapes[name]
        o = self.offsets[_NAMES.index(name)]
        n = 1
        for d in shp:
            n *= d
        nbytes = n * torch.tensor([], dtype=dt).element_size()
        return self.buf[o:o + nbytes].view(dt).view(shp)


def _layer_args(logits, xq, xs, w1, w2, k, e0, n_local, shared, flags, out, hTq, hTs, epi=None):
    T, E_tot = logits.shape
    H = xq.shape[1]
    args = moe_layer_args()
    args.logits, args.T, args.E_tot, args.k = _p(logits), T, E_tot, k
    args.e0, args.E_loc = e0, n_local
    args.xq, args.xs, args.H, args.I = _p(xq), _p(xs), H, w1.N // 2
    args.w1, args.w2 = C.pointer(w1.desc), C.pointer(w2.desc)
    if shared is not None:
        args.shared_w1, args.shared_w2 = C.pointer(shared[0].desc), C.pointer(shared[1].desc)
    args.flags = flags
    args.hTq, args.hTs = _p(hTq), _p(hTs)
    args.out = _p(out)
    if epi is not None:
        args.epi = C.pointer(epi.desc)
    return args


def moe_layer(logits, xq, xs, w1: PackedWeights, w2: PackedWeights, k: int, e0: int = 0,
              n_local: int | None = None, shared=None, flags: int = 0, out=None, ws=None,
              hTq=None, hTs=None, epi: Epilogue | None = None, stream=None):
    """Whole layer. shared = (PackedWeights W1, PackedWeights W2) or None.
    Returns out (bf16 bits as uint16 [T, H])."""
    _dev(logits, torch.float32, "logits")
    _dev(xq, torch.uint8, "xq")
    _dev(xs, torch.uint8, "xs")
    T, E_tot = logits.shape
    H = xq.shape[1]
    I = w1.N // 2
    n_local = w1.G if n_local is None else n_local
    s = 1 if shared is not None else 0
    with _on(stream):
        if out is None:
            out = torch.empty((T, H), dtype=torch.uint16, device=xq.device)
        if ws is None:
            ws = LayerWorkspace(T, E_tot, k, n_local, H, I, bool(s), flags, device=xq.device)
        args = _layer_args(logits, xq, xs, w1, w2, k, e0, n_local, shared, flags, out, hTq, hTs, epi)
        _check(lib.moe_layer(C.byref(args), _p(ws.buf), ws.nbytes, _stream()), "moe_layer")
    return out


def moe_layer_noalloc(logits, xq, xs, w1: PackedWeights, w2: PackedWeights, k: int, e0: int = 0,
                      n_local: int | None = None, shared=None, flags: int = 0, out=None,
                      hTq=None, hTs=None, stream=None):
    """moe_layer with the library's fixed per-GPU workspace (no workspace
    argument, nothing allocated by the library). `out` must be given when the
    call must not allocate either; calls overlapping on one GPU race."""
    _dev(logits, torch.float32, "logits")
    _dev(xq, torch.uint8, "xq")
    _dev(xs, torch.uint8, "xs")
    T = logits.shape[0]
    n_local = w1.G if n_local is None else n_local
    with _on(stream):
        if out is None:
            out = torch.empty((T, xq.shape[1]), dtype=torch.uint16, device=xq.device)
        args = _layer_args(logits, xq, xs, w1, w2, k, e0, n_local, shared, flags, out, hTq, hTs)
        _check(lib.moe_layer_noalloc(C.byref(args), _stream()), "moe_layer_noalloc")
    return out


def layer(xq, xs, logits, w1: PackedWeights, w2: PackedWeights, k: int, e0: int = 0,
          n_local: int | None = None, shared=None, flags: int = 0, out=None, **kw):
    """moe_layer with the argument order of the activation-first call form
    (x codes, x scales, router logits, weights, top-k)."""
    return moe_layer(logits, xq, xs, w1, w2, k, e0, n_local, shared, flags, out=out, **kw)
