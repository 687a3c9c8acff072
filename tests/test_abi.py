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
    offs = (C.c_size_t * 12)()
    assert lib.moe_layer_workspace_offsets(T, E, k, El, H, I, 0, 0, offs) == 12
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
