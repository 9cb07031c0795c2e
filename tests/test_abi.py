"""The C ABI on the CPU: the library loads, exports every function that
include/dmm.h declares, and rejects invalid arguments with DMM_EINVAL before
making any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dmm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)) - {"if"})


@pytest.fixture(scope="module")
def L():
    import dense_matmul_amd as dmm

    if not os.path.exists(dmm.LIB_PATH):
        from dense_matmul_amd import build

        build.build()
    return dmm.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("quantize_per_token", "quantize_per_token_bf16", "preshuffle_b", "gemm_a8w8_ptpc", "gemm_a8w8_ptpc_tile", "gemm_a8w8_ptpc_gathered",
              "gemm_a8w8_blockscale", "gemm_a8w8_blockscale_tile",
              "gemm_a8w8_mxfp8", "gemm_a8w8_mxfp8_tile",
              "gemm_bf16", "gemm_bf16_tile", "quantize_blockscale_a", "quantize_blockscale_b", "quantize_mxfp8", "dmm_status_str",
              "dmm_last_error"):
        assert f in names, f
    # the benchmark's calibration kernel lives in its own library, not in the boundary
    assert not any("ceiling" in f or "calib" in f for f in names)


def test_library_exports_every_declared_function(L):
    for name in declared_functions():
        assert hasattr(L, name), f"libdmm.so does not export {name}"


def test_binding_declares_every_signature(L):
    """Every function the binding exports has its ctypes argument types set
    (an unset one would pass 64-bit sizes as 32-bit ints), and the list is
    exactly the header's."""
    import dense_matmul_amd as dmm

    assert set(dmm.EXPORTS) == set(declared_functions())
    for name in dmm.EXPORTS:
        assert getattr(L, name).argtypes is not None, name


def test_status_strings(L):
    assert L.dmm_status_str(0) == b"DMM_OK"
    assert L.dmm_status_str(1) == b"DMM_EINVAL"
    assert L.dmm_status_str(99) == b"DMM_UNKNOWN"


ALIGNED = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("m,n,k,why", [
    (0, 256, 256, "m must be"), (64, 24, 256, "n must be"), (64, 8, 256, "n must be"), (64, 256, 200, "k must be"),
    (64, 256, 0, "k must be"), (1 << 22, 1024, 1024, "too large"), (64, 1 << 22, 1024, "too large"),
])
def test_gemm_shape_rules(L, m, n, k, why):
    for fn in (L.gemm_a8w8_ptpc, L.gemm_a8w8_blockscale, L.gemm_a8w8_mxfp8):
        assert fn(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, m, n, k, None) == 1
        assert why in L.dmm_last_error().decode()


@pytest.mark.parametrize("name", ["gemm_a8w8_ptpc_tile", "gemm_a8w8_blockscale_tile", "gemm_a8w8_mxfp8_tile"])
def test_tile_rule(L, name):
    """tile is 0 (auto), 1 (the wide tile) or 2 (the half-size one), and 3
    (128 x 128) for ptpc; anything else is an argument error, reported
    before any HIP call."""
    f = getattr(L, name)
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_void_p]
    for tile in (-1, 4 if name == "gemm_a8w8_ptpc_tile" else 3, 256):
        assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 64, 256, 256, tile, None) == 1
        assert b"tile must be" in L.dmm_last_error()
    # shape rules apply as for the call without a tile
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 64, 24, 256, 2, None) == 1


@pytest.mark.parametrize("m,src_rows,nchunks,own,spin,why", [
    (4096, 1000, 1, 0, 10, "src_rows must be"),       # not a multiple of 256
    (4096, 1024, 3, 0, 10, "src_rows must be"),       # 1024 rows do not split into 3 chunks of whole tiles
    (4096, 1536, 1, 0, 10, "m must be a multiple"),
    (4096, 1024, 1, 4, 10, "own must name"),
    (4096, 1024, 1, -1, 10, "own must name"),
    (65 * 256, 256, 1, 0, 10, "at most 64 bands"),
    (4096, 1024, 0, 0, 10, "nchunks must be"),
    (4096, 1024, 1, 0, -1, "spin_limit"),
])
def test_gathered_rules(L, m, src_rows, nchunks, own, spin, why):
    f = L.gemm_a8w8_ptpc_gathered
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                                                 ctypes.c_int, ctypes.c_uint32, ctypes.c_int64,
                                                                 ctypes.c_void_p, ctypes.c_void_p]
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, m, 256, 256, ALIGNED, src_rows, nchunks, own, 7, spin,
             ALIGNED, None) == 1
    assert why in L.dmm_last_error().decode()
    # flags and status must be given
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 4096, 256, 256, None, 1024, 1, 0, 7, 10, ALIGNED,
             None) == 1
    assert b"flags" in L.dmm_last_error()


def test_bf16_tile_rule(L):
    f = L.gemm_bf16_tile
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_void_p]
    for tile in (-1, 3):
        assert f(ALIGNED, ALIGNED, ALIGNED, 64, 256, 256, tile, None) == 1
        assert b"tile must be" in L.dmm_last_error()
    assert f(ALIGNED, ALIGNED, ALIGNED, 64, 24, 256, 2, None) == 1


def test_gemm_pointer_rules(L):
    bad = ctypes.c_void_p((1 << 20) + 4)
    assert L.gemm_a8w8_ptpc(None, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 64, 256, 256, None) == 1
    assert b"a:" in L.dmm_last_error()
    assert L.gemm_a8w8_ptpc(ALIGNED, bad, ALIGNED, ALIGNED, ALIGNED, 64, 256, 256, None) == 1
    assert b"b:" in L.dmm_last_error()
    assert L.gemm_bf16(ALIGNED, ALIGNED, None, 64, 256, 256, None) == 1


def test_quantiser_and_preshuffle_rules(L):
    assert L.quantize_per_token(ALIGNED, ALIGNED, ALIGNED, 0, 256, None) == 1
    assert L.quantize_per_token(ALIGNED, ALIGNED, ALIGNED, 4, 17, None) == 1
    L.quantize_per_token_bf16.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]
    assert L.quantize_per_token_bf16(ALIGNED, ALIGNED, ALIGNED, 4, 24, None) == 1
    assert L.quantize_per_token_bf16(ALIGNED, ALIGNED, ALIGNED, 0, 32, None) == 1
    assert L.quantize_blockscale_a(ALIGNED, ALIGNED, ALIGNED, 4, 100, None) == 1
    assert L.quantize_blockscale_b(ALIGNED, ALIGNED, ALIGNED, 20, 128, None) == 1
    assert L.quantize_mxfp8(ALIGNED, ALIGNED, ALIGNED, 4, 96, None) == 1
    assert L.preshuffle_b(ALIGNED, ALIGNED, 24, 128, None) == 1
    # overlapping source and destination
    assert L.preshuffle_b(ALIGNED, ctypes.c_void_p((1 << 20) + 256), 16, 128, None) == 1
    assert b"overlap" in L.dmm_last_error()
    assert L.gemm_bf16(ALIGNED, ALIGNED, ALIGNED, 4, 16, 96, None) == 1
