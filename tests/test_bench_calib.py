"""The benchmark's matrix-op calibration kernel (libdmm_calib.so, built beside
libdmm but not part of its C ABI): argument rules on the CPU, and on the GPU
that every variant runs on every compute unit, reports its FLOPs and is
deterministic."""
import ctypes
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

ALIGNED = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bench.CALIB_LIB):
        from dense_matmul_amd import build

        build.build()
    return bench.calib_lib()


def test_calibration_is_not_in_the_product_library():
    import dense_matmul_amd as dmm

    if not os.path.exists(dmm.LIB_PATH):
        pytest.skip("libdmm.so not built")
    lib = ctypes.CDLL(dmm.LIB_PATH)
    for name in ("calib_mfma_ceiling_fp8", "dmm_mfma_ceiling_fp8"):
        assert not hasattr(lib, name), name


@pytest.mark.parametrize("frag,frag_bytes,out_len,iters,wps,var,why", [
    (ALIGNED, 1 << 20, 16, 1, 1, 0, "frag must hold"), (ALIGNED, 1 << 21, 0, 1, 1, 0, "out_len"),
    (ALIGNED, 1 << 21, 16, 0, 1, 0, "iters"), (ALIGNED, 1 << 21, 16, (1 << 20) + 1, 1, 0, "iters"),
    (ALIGNED, 1 << 21, 16, 1, 3, 0, "waves_per_simd"), (ALIGNED, 1 << 21, 16, 1, 0, 0, "waves_per_simd"),
    (ALIGNED, 1 << 21, 16, 1, 1, 12, "variant"), (ALIGNED, 1 << 21, 16, 1, 1, -1, "variant"),
    (ctypes.c_void_p((1 << 20) + 4), 1 << 21, 16, 1, 1, 0, "frag: pointer"),
    (None, 1 << 21, 16, 1, 1, 0, "frag: pointer"),
])
def test_calibration_rules(L, frag, frag_bytes, out_len, iters, wps, var, why):
    """The entry point checks its arguments before any HIP call."""
    st = L.calib_mfma_ceiling_fp8(frag, frag_bytes, ALIGNED, out_len, iters, wps, var, None, None)
    assert st == 1, st
    assert why in L.calib_last_error().decode()


@pytest.mark.gpu
@pytest.mark.parametrize("variant", list(bench.CALIB_VARIANTS))
@pytest.mark.parametrize("wps", [1, 2])
def test_calibration_kernel_runs_and_is_deterministic(L, wps, variant):
    """Every compute unit runs it, the FLOPs of the launch are as stated, and
    its accumulators are finite and equal across two launches; the variants
    of one matrix-op shape give equal sums (the extra instructions never feed
    the matrix ops)."""
    import torch

    print("[case] calibration kernel, waves per SIMD", wps, "variant", variant, flush=True)
    g = torch.Generator().manual_seed(5)
    frag = torch.randint(0, 0x7F, (1 << 21,), dtype=torch.uint8, generator=g).to("cuda:0")  # finite codes
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out1, flops = bench.mfma_ceiling_fp8(frag, 3, wps, variant)
    out2, _ = bench.mfma_ceiling_fp8(frag, 3, wps, variant)
    ref, _ = bench.mfma_ceiling_fp8(frag, 3, wps, "w32_plain" if variant.startswith("w32") else "plain")
    torch.cuda.synchronize()
    assert flops == 2.0 * 16 * 16 * 128 * 16 * 3 * cus * 4 * wps
    used = cus * 256 * wps
    assert torch.isfinite(out1[:used]).all()
    assert torch.equal(out1[:used], out2[:used])
    assert torch.equal(out1[:used], ref[:used])
    assert (out1[:used] != 0).any()
