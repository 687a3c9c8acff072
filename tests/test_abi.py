"""The C-ABI library loads and exports every symbol include/moe.h declares;
argument validation answers without a GPU (no compute calls here)."""
import ctypes as C
import os
import re

import pytest

from routed_grouped_gemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    lib = _lib.load()
    names = _declared()
    assert len(names) >= 16, names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"
    assert set(_lib.SIGNATURES) == set(names)


def test_version_and_status_strings():
    lib = _lib.load()
    assert b"gfx950" in lib.moe_version()
    for st in range(6):
        assert lib.moe_status_string(st)
    assert lib.moe_status_string(99) == b"unknown status"


def test_route_validation():
    lib = _lib.load()
    assert lib.moe_route(None, 4, 8, 0, 0, None, None, None) == _lib.MOE_ERR_SHAPE      # k = 0
    assert lib.moe_route(None, 4, 8, 9, 0, None, None, None) == _lib.MOE_ERR_SHAPE      # k > E
    assert lib.moe_route(None, 4, 4096, 8, 0, None, None, None) == _lib.MOE_ERR_SHAPE   # E > 2048
    assert lib.moe_route(None, 4, 64, 33, 0, None, None, None) == _lib.MOE_ERR_SHAPE    # k > 32
    assert lib.moe_route(None, 4, 8, 2, 0, None, None, None) == _lib.MOE_ERR_NULL
    assert lib.moe_route(None, 0, 8, 2, 0, None, None, None) == _lib.MOE_OK              # T = 0


def test_hbm_read_probe_validation():
    lib = _lib.load()
    assert lib.moe_hbm_read_probe(None, 24, None, None) == _lib.MOE_ERR_SHAPE             # not whole chunks
    assert lib.moe_hbm_read_probe(None, (1 << 31) + 16, None, None) == _lib.MOE_ERR_SHAPE  # over 2 GiB
    assert lib.moe_hbm_read_probe(None, 1 << 20, None, None) == _lib.MOE_ERR_NULL
    assert lib.moe_hbm_read_probe(None, 0, None, None) == _lib.MOE_OK                      # nothing to read


def test_permute_validation():
    lib = _lib.load()
    args = lambda T, k, e0, El, s, H: (None, None, T, k, e0, El, s, None, None, H,  # noqa: E731
                                       None, None, None, None, None, None, None, None, None, 0, None)
    assert lib.moe_permute(*args(4, 8, 0, 32, 0, 7168)) == _lib.MOE_ERR_NULL
    assert lib.moe_permute(*args(4, 32, 0, 32, 1, 7168)) == _lib.MOE_ERR_SHAPE    # k + s > 32
    assert lib.moe_permute(*args(4, 8, 0, 32, 0, 7000)) == _lib.MOE_ERR_SHAPE     # H % 256
    assert lib.moe_permute(*args(4, 8, 2040, 32, 0, 7168)) == _lib.MOE_ERR_SHAPE  # e0 + E_loc > 2048
    assert lib.moe_permute(*args(4, 8, 0, 0, 0, 7168)) == _lib.MOE_ERR_SHAPE      # no local experts


def test_sizes_are_pure_host_functions():
    lib = _lib.load()
    # FP4: 64-row unit x 128-K tile = 4 KiB data + scales 1 KiB per 4 K-tiles
    assert lib.moe_prepacked_size(1, 64, 128, _lib.MOE_FMT_MXFP4) == 4096 + 1024
    assert lib.moe_prepacked_size(1, 64, 512, _lib.MOE_FMT_MXFP8) == 4 * 8192 + 1024
    assert lib.moe_prepacked_size(2, 64, 128, _lib.MOE_FMT_MXFP4) == 2 * (4096 + 1024)
    assert lib.moe_prepacked_size(1, 60, 128, 0) == 0 and lib.moe_prepacked_size(1, 64, 100, 0) == 0
    assert lib.moe_transposed_ld(98304, 64) == (98304 + 31 * 64 + 31) // 32 * 32
    # layer workspace holds at least every intermediate for R_max rows
    T, E, k, El, H, I = 128, 256, 8, 32, 7168, 2048
    R = T * k
    need = R * I + R * I // 32 + 2 * R * H
    assert lib.moe_layer_workspace_size(T, E, k, El, H, I, 0, 0) >= need
    offs = (C.c_size_t * 13)()
    assert lib.moe_layer_workspace_offsets(T, E, k, El, H, I, 0, 0, offs) == 13
    assert all(o % 256 == 0 for o in offs) and list(offs) == sorted(offs)


def test_weight_and_layer_validation():
    lib = _lib.load()
    w = _lib.moe_weights(_lib.MOE_FMT_MXFP4, 8, 512, 512, 1, 0, 0x1000,
                         lib.moe_prepacked_size(8, 512, 512, 0))
    args = _lib.moe_layer_args()
    args.T, args.E_tot, args.k, args.e0, args.E_loc, args.H, args.I = 16, 8, 2, 0, 8, 512, 256
    args.w1 = C.pointer(w)
    w2 = _lib.moe_weights(_lib.MOE_FMT_MXFP4, 8, 512, 256, 0, 0, 0x1000,
                          lib.moe_prepacked_size(8, 512, 256, 0))
    args.w2 = C.pointer(w2)
    # w1 has N = 512 = 2I but K = 512 = H: valid; missing logits -> NULL
    assert lib.moe_layer(C.byref(args), None, 0, None) == _lib.MOE_ERR_NULL
    args.I = 200                                   # I % 128 != 0
    assert lib.moe_layer(C.byref(args), None, 0, None) == _lib.MOE_ERR_SHAPE
    args.I = 256
    w.bytes = 10                                   # undersized weight buffer
    assert lib.moe_layer(C.byref(args), None, 0, None) == _lib.MOE_ERR_WORKSPACE
    w.bytes = lib.moe_prepacked_size(8, 512, 512, 0)
    w.fmt = 7
    assert lib.moe_layer(C.byref(args), None, 0, None) == _lib.MOE_ERR_UNSUPPORTED
    w.fmt = 0
    args.flags = _lib.MOE_W1_WRITE_TRANSPOSE       # transposed copy without buffers
    assert lib.moe_layer(C.byref(args), None, 0, None) == _lib.MOE_ERR_NULL
    args.flags = 0
    args.T = 0                                     # nothing to do
    assert lib.moe_layer(C.byref(args), None, 0, None) == _lib.MOE_OK


def test_binding_requires_device_tensors():
    torch = pytest.importorskip("torch")
    import routed_grouped_gemm_amd as moe
    with pytest.raises(moe.MoeError):
        moe.moe_route(torch.zeros((2, 8), dtype=torch.float32), 2)


def _w(fmt, G, N, K, is_w1):
    lib = _lib.load()
    return _lib.moe_weights(fmt, G, N, K, is_w1, 0, 0x1000, lib.moe_prepacked_size(G, N, K, fmt))


def test_grouped_w1_status_paths():
    """Every status moe_grouped_w1 can return from its scalar checks (nothing
    is launched: all of them fail before the first enqueue)."""
    lib = _lib.load()
    F = 0x1000                                      # stands for a device pointer; never dereferenced
    I, H, G, R = 256, 512, 4, 64
    w = _w(_lib.MOE_FMT_MXFP4, G, 2 * I, H, 1)

    def call(w1=w, counts=F, offsets=F, off32=None, row_w=F, xq=F, xs=F, row_src=None, x_rows=R,
             R_max=R, H=H, I=I, G=G, flags=0, hq=F, hs=F, hTq=None, hTs=None, ws=F, ws_bytes=1 << 30):
        return lib.moe_grouped_w1(C.byref(w1), None, counts, offsets, off32, row_w, xq, xs, row_src,
                                  x_rows, R_max, H, I, G, None, flags, hq, hs, hTq, hTs, ws, ws_bytes, None)

    both = _lib.MOE_GEMM_STREAMED | _lib.MOE_GEMM_TILED
    assert call(flags=both) == _lib.MOE_ERR_UNSUPPORTED
    # any two of the three kernel families
    assert call(flags=_lib.MOE_GEMM_PASS | _lib.MOE_GEMM_STREAMED) == _lib.MOE_ERR_UNSUPPORTED
    assert call(flags=_lib.MOE_GEMM_PASS | _lib.MOE_GEMM_TILED) == _lib.MOE_ERR_UNSUPPORTED
    assert call(I=200) == _lib.MOE_ERR_SHAPE                                     # I % 128
    assert call(H=500) == _lib.MOE_ERR_SHAPE                                     # H % 256
    assert call(x_rows=0) == _lib.MOE_ERR_SHAPE
    assert call(R_max=1 << 23, x_rows=1 << 23, I=256) == _lib.MOE_ERR_SHAPE      # R_max * I >= 2^31
    assert call(x_rows=(1 << 31) // H, row_src=F) == _lib.MOE_ERR_SHAPE          # x_rows * H >= 2^31
    # I * ldT >= 2^31 with the transposed copy (ldT ~ R_max)
    assert call(R_max=600000, x_rows=600000, flags=_lib.MOE_W1_WRITE_TRANSPOSE, off32=F, hTq=F,
                hTs=F, H=256) == _lib.MOE_ERR_SHAPE
    assert call(x_rows=R // 2) == _lib.MOE_ERR_SHAPE                             # ungrouped rows need row_src
    bad = _w(_lib.MOE_FMT_MXFP4, G + 1, 2 * I, H, 1)
    assert call(w1=bad) == _lib.MOE_ERR_SHAPE                                    # weights for other groups
    assert call(hq=None) == _lib.MOE_ERR_NULL
    assert call(row_w=None) == _lib.MOE_ERR_NULL                                 # weight applied in W1
    assert call(flags=_lib.MOE_W1_WRITE_TRANSPOSE) == _lib.MOE_ERR_NULL          # no hT buffers
    assert call(ws=None, ws_bytes=0) == _lib.MOE_ERR_WORKSPACE


def test_grouped_w2_status_paths():
    lib = _lib.load()
    F = 0x1000
    I, H, G, R = 256, 512, 4, 64
    w = _w(_lib.MOE_FMT_MXFP8, G, H, I, 0)

    def call(w2=w, counts=F, R_max=R, H=H, I=I, G=G, flags=0, y=F, ws=F, ws_bytes=1 << 30):
        return lib.moe_grouped_w2(C.byref(w2), None, counts, F, F, F, R_max, H, I, G, flags, y, ws,
                                  ws_bytes, None)

    assert call(flags=_lib.MOE_GEMM_STREAMED | _lib.MOE_GEMM_TILED) == _lib.MOE_ERR_UNSUPPORTED
    assert call(flags=_lib.MOE_GEMM_PASS | _lib.MOE_GEMM_TILED) == _lib.MOE_ERR_UNSUPPORTED
    assert call(flags=_lib.MOE_W1_WRITE_TRANSPOSE) == _lib.MOE_ERR_UNSUPPORTED   # no W1 flags here
    assert call(I=4224) == _lib.MOE_ERR_SHAPE                                    # I > 4096
    assert call(R_max=1 << 23) == _lib.MOE_ERR_SHAPE                             # R_max * I >= 2^31
    assert call(G=0) == _lib.MOE_ERR_SHAPE
    assert call(w2=_w(_lib.MOE_FMT_MXFP8, G, H, 2 * I, 0)) == _lib.MOE_ERR_SHAPE  # K != I
    assert call(y=None) == _lib.MOE_ERR_NULL
    assert call(counts=None) == _lib.MOE_ERR_NULL
    assert call(ws=None, ws_bytes=0) == _lib.MOE_ERR_WORKSPACE


def test_combine_validation():
    lib = _lib.load()
    assert lib.moe_combine(None, None, None, 4, 0, 512, None, None) == _lib.MOE_ERR_SHAPE    # no slots
    assert lib.moe_combine(None, None, None, 4, 33, 512, None, None) == _lib.MOE_ERR_SHAPE   # > 32 slots
    assert lib.moe_combine(None, None, None, 4, 8, 500, None, None) == _lib.MOE_ERR_SHAPE    # H % 8
    assert lib.moe_combine(None, None, None, 4, 8, 512, None, None) == _lib.MOE_ERR_NULL
    assert lib.moe_combine(None, None, None, 0, 8, 512, None, None) == _lib.MOE_OK           # T = 0


def test_layer_rejects_oversized_prefill_before_enqueueing():
    """A prefill whose h would pass 2^31 bytes (T = 131072, k = 8, I = 2048)
    is refused from its scalars alone: the call passes a NULL stream and fake
    pointers, so any enqueue would fault instead of returning a status."""
    lib = _lib.load()
    w1 = _w(_lib.MOE_FMT_MXFP8, 64, 4096, 2048, 1)
    w2 = _w(_lib.MOE_FMT_MXFP8, 64, 2048, 2048, 0)
    args = _lib.moe_layer_args()
    args.logits = args.xq = args.xs = args.out = 0x1000
    args.T, args.E_tot, args.k, args.e0, args.E_loc, args.H, args.I = 131072, 64, 8, 0, 64, 2048, 2048
    args.w1, args.w2 = C.pointer(w1), C.pointer(w2)
    assert lib.moe_layer(C.byref(args), 0x1000, 1 << 40, None) == _lib.MOE_ERR_SHAPE
    args.flags = _lib.MOE_GEMM_STREAMED | _lib.MOE_GEMM_TILED
    args.T = 16
    assert lib.moe_layer(C.byref(args), 0x1000, 1 << 40, None) == _lib.MOE_ERR_UNSUPPORTED


def test_noalloc_rejects_workspace_beyond_its_array():
    """The fixed workspace holds MOE_NOALLOC_SCRATCH_BYTES; a layer needing more
    (the 16K-token prefill) is refused from its scalars, before any HIP call."""
    lib = _lib.load()
    T, E, k, El, H, I = 16384, 64, 6, 64, 2048, 1408
    assert lib.moe_layer_workspace_size(T, E, k, El, H, I, 0, 0) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    w1 = _w(_lib.MOE_FMT_MXFP8, El, 2 * I, H, 1)
    w2 = _w(_lib.MOE_FMT_MXFP8, El, H, I, 0)
    args = _lib.moe_layer_args()
    args.logits = args.xq = args.xs = args.out = 0x1000
    args.T, args.E_tot, args.k, args.e0, args.E_loc, args.H, args.I = T, E, k, 0, El, H, I
    args.w1, args.w2 = C.pointer(w1), C.pointer(w2)
    assert lib.moe_layer_noalloc(C.byref(args), None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_layer_noalloc(None, None) == _lib.MOE_ERR_NULL
    args.T = 0                                     # nothing to enqueue: no workspace needed
    assert lib.moe_layer_noalloc(C.byref(args), None) == _lib.MOE_OK
    args.T, args.I = 16, 200                       # other argument errors come from moe_layer's checks
    assert lib.moe_layer_noalloc(C.byref(args), None) == _lib.MOE_ERR_SHAPE


def test_backward_and_epilogue_status_paths():
    lib = _lib.load()
    F = 0x1000
    I, H, G, R = 256, 512, 4, 64
    w2t = _w(_lib.MOE_FMT_MXFP8, G, I, H, 0)
    ok_epi = _lib.moe_epilogue(_lib.MOE_ACT_GEGLU, 1.0, 0.0, 0, None, None)

    def call(w=w2t, epi=None, flags=0, pre=F, dq=F, row_w=F, dw=F, I=I, R_max=R, ws_bytes=1 << 30,
             dTq=None, off32=None):
        return lib.moe_grouped_w1_backward(C.byref(w), None, F, F, off32, row_w, F, F, F, R, pre, R_max, H,
                                           I, G, None if epi is None else C.byref(epi), flags, dq, F, dTq, F,
                                           dw, F, ws_bytes, None)

    assert lib.moe_backward_workspace_size(R, G, H, I) >= R * (I // 64) * 4
    assert call(flags=_lib.MOE_ROUTE_RENORM) == _lib.MOE_ERR_UNSUPPORTED
    assert call(epi=_lib.moe_epilogue(7, 1.0, 0.0, 0, None, None)) == _lib.MOE_ERR_UNSUPPORTED
    assert call(epi=_lib.moe_epilogue(0, 0.0, 0.0, 0, None, None)) == _lib.MOE_ERR_SHAPE     # beta = 0
    assert call(epi=_lib.moe_epilogue(0, 1.0, -1.0, 0, None, None)) == _lib.MOE_ERR_SHAPE    # limit < 0
    assert call(epi=_lib.moe_epilogue(0, float("nan"), 0.0, 0, None, None)) == _lib.MOE_ERR_SHAPE
    assert call(I=200) == _lib.MOE_ERR_SHAPE
    assert call(R_max=1 << 21, I=256) == _lib.MOE_ERR_SHAPE                    # R_max * 2I bytes >= 2^31
    assert call(w=_w(_lib.MOE_FMT_MXFP8, G, 2 * I, H, 0)) == _lib.MOE_ERR_SHAPE  # N must be I
    assert call(pre=None, epi=ok_epi) == _lib.MOE_ERR_NULL
    assert call(dq=None) == _lib.MOE_ERR_NULL
    assert call(row_w=None) == _lib.MOE_ERR_NULL                               # dw needs the weights
    assert call(flags=_lib.MOE_W1_WRITE_TRANSPOSE) == _lib.MOE_ERR_NULL        # no transposed buffers
    assert call(ws_bytes=0) == _lib.MOE_ERR_WORKSPACE
    # the forward's epilogue is validated the same way
    w1 = _w(_lib.MOE_FMT_MXFP4, G, 2 * I, H, 1)
    bad = _lib.moe_epilogue(3, 1.0, 0.0, 0, None, None)
    assert lib.moe_grouped_w1(C.byref(w1), None, F, F, None, F, F, F, None, R, R, H, I, G, C.byref(bad), 0,
                              F, F, None, None, F, 1 << 30, None) == _lib.MOE_ERR_UNSUPPORTED
