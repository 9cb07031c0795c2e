"""The benchmark's calibration kernels (libdmm_calib.so, built beside libdmm
but not part of its C ABI): argument rules on the CPU, and on the GPU that
every matrix-op variant runs on every compute unit, reports its FLOPs and is
deterministic, and that the memory-rate kernel writes what it is asked to and
reports plausible rates."""
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
    for name in ("calib_mfma_ceiling_fp8", "dmm_mfma_ceiling_fp8", "calib_memory_rate"):
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


@pytest.mark.parametrize("buf,buf_bytes,region,iters,kind,grid,why", [
    (None, 1 << 30, 1 << 16, 1, 0, 1, "buf: pointer"), (ctypes.c_void_p((1 << 20) + 8), 1 << 30, 1 << 16, 1, 0, 1, "buf: pointer"),
    (ALIGNED, 1 << 30, 1 << 16, 1, 4, 1, "kind"), (ALIGNED, 1 << 30, 1 << 16, 1, -1, 1, "kind"),
    (ALIGNED, 1 << 30, 1 << 15, 1, 0, 1, "region"), (ALIGNED, 1 << 30, 3 << 16, 1, 0, 1, "region"),
    (ALIGNED, 1 << 30, 1 << 20, 1, 3, 1, "region"), (ALIGNED, 1 << 30, (1 << 30) * 2, 1, 0, 1, "region"),
    (ALIGNED, 1 << 30, 1 << 16, 0, 0, 1, "iters"), (ALIGNED, 1 << 30, 1 << 16, (1 << 16) + 1, 0, 1, "iters"),
])
def test_memory_rate_rules(L, buf, buf_bytes, region, iters, kind, grid, why):
    """The memory-rate entry point checks its arguments before any HIP call."""
    st = L.calib_memory_rate(buf, buf_bytes, region, iters, kind, 0, grid, ALIGNED, None)
    assert st == 1, st
    assert why in L.calib_last_error().decode()


@pytest.mark.gpu
def test_memory_rate_kernel_writes_its_region_and_reports_rates(L):
    """The store kinds write exactly their workgroups' regions (a poisoned
    buffer keeps its poison past grid * region), the epilogue pattern covers
    the rows it claims, and every kind reports a positive, finite rate below
    the L1's 64 bytes per cycle per CU for HBM-bound regions."""
    import torch

    print("[case] memory-rate kernel", flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    region = 4 << 20
    buf = torch.full((cus * region + (1 << 20),), 0xEE, dtype=torch.uint8, device="cuda:0")
    bench.memory_rate(torch, buf, region, "stores_lines", grid=8, iters=4, launches=1)
    torch.cuda.synchronize()
    b = buf.view(torch.int32)
    lines = b[: 8 * region // 4].view(8, region // 4)
    # kind 2 writes {lane, wave, workgroup, 7} per 16 bytes over the region's first 4 waves x 16 x 4 KiB
    assert (lines[:, 3::4][:, : 4 * 4 * 16 * 1024 // 16] == 7).all()
    assert (buf[8 * region:] == 0xEE).all()
    for kind in bench.MEMORY_KINDS:
        per_cu, tbs = bench.memory_rate(torch, buf[: cus * region], region, kind, iters=16, launches=2)
        print("[stats]", kind, per_cu, tbs, flush=True)
        assert 0.5 < per_cu < 64.0 and 0.05 < tbs < 40.0, (kind, per_cu, tbs)


def test_code_text_drops_comments_and_blank_space_only():
    src = "int a = 1; // the count\n/* a block\n   comment */\tint  b = a /2;\n"
    assert bench.code_text(src) == "int a = 1; int b = a /2;"
    assert bench.code_text("x = y;") != bench.code_text("x = z;")


def test_committed_traffic_profile_is_for_the_current_kernel():
    # the bench reports roofline.traffic only from a counter summary taken on
    # the GEMM sources as they are; a kernel change needs new counter runs
    traffic = bench.traffic_from_profiles("gemm_a8w8_ptpc")
    assert traffic is not None, "profiles/gemm_a8w8_ptpc_traffic.json was taken on other kernel sources"
    assert 5e8 < traffic < 5e9
