"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times (the library's own tile choice, one call per GEMM).

The inputs are the workloads' seeded N(0,1) operands quantised on the host
by the oracle's quantisers (the GPU quantisers are tested bitwise against
the same functions elsewhere), so no expected value comes from the GPU.
Each GEMM runs 20 times, each launch into a freshly NaN-poisoned C followed
by a canary (mori PR 785, Test: NaN-poison before each launch; aiter PR
6539, Test Plan: 20 launches per shape): every launch must equal the first
bitwise (compared on the device), launch 0 must leave no NaN, no launch may
touch the canary, and launch 0's sampled rows (every row of the first and
last 256-row tiles plus one per 64-row band) must meet the acceptance rule
against the oracle, which computes only those rows.  The
smaller workloads (512x1024x256, 4096x7168x256, 16384x7168x512,
2048x1168x1792, the bf16 GEMM) are tested in full elsewhere."""
import numpy as np
import pytest
import torch

import oracle
from dense_matmul_amd import inputs
from oracle import tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

FULL = ["ptpc_32768x7168x1792", "blockscale_16384x7168x2048", "mxfp8_32768x7168x1792", "mxfp8_16384x7168x2048",
        "ptpc_gathered_32768x6288x7168", "ptpc_gathered_32768x3648x7168"]
MODE_ID = {"ptpc": 0, "blockscale": 1, "mxfp8": 2}
LAUNCHES = 20


@pytest.fixture(scope="module")
def dmm():
    import dense_matmul_amd as d

    d.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return d


def quantise(mode, x, side):
    if mode == "ptpc":
        return oracle.quantize_per_token(x)
    if mode == "blockscale":
        return oracle.quantize_blockscale_a(x) if side == "a" else oracle.quantize_blockscale_b(x)
    return oracle.quantize_mxfp8(x)


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(dmm, name):
    mode, m, n, k, seed_a, seed_b = inputs.WORKLOADS[name]
    print("[case] full size", name, flush=True)
    qa, sa = quantise(mode, inputs.operand_a(m, k, seed_a), "a")
    qb, sb = quantise(mode, inputs.normal((n, k), seed_b), "b")
    a, s_a, s_b = (torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in (qa, sa, sb))
    b_shuf = dmm.preshuffle_b(torch.from_numpy(qb).to(DEV))
    fn = {"ptpc": dmm.gemm_a8w8_ptpc, "blockscale": dmm.gemm_a8w8_blockscale, "mxfp8": dmm.gemm_a8w8_mxfp8}[mode]
    buf = torch.empty(m * n + 2048, dtype=torch.bfloat16, device=DEV)
    c = buf[: m * n].view(m, n)
    canary = buf[m * n:].view(torch.int16)
    first = None
    for i in range(LAUNCHES):
        buf.fill_(float("nan"))
        canary.fill_(0x5A5A)
        fn(a, b_shuf, s_a, s_b, out=c)
        if first is None:
            first = c.clone()
            assert not torch.isnan(first).any().item(), f"{name}: unwritten elements"
        else:
            same = torch.equal(c.view(torch.int16), first.view(torch.int16))
            assert same, f"{name}: launch {i} differs from launch 0 in " \
                         f"{int((c.view(torch.int16) != first.view(torch.int16)).sum())} elements"
        assert bool((canary == 0x5A5A).all().item()), f"{name}: launch {i} wrote past the end of C"
    print(f"[bitwise] {name}: {LAUNCHES} launches identical", flush=True)
    rows = inputs.rows_sample(m, seed=m + n + k)
    got = first.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    ref = oracle.gemm_a8w8(MODE_ID[mode], qa, qb, sa, sb, rows=rows)
    stats = tolerance.check(got, ref, f"{name} sampled rows", mode=mode, operands=(qa, qb, sa, sb), rows=rows)
    print("[stats]", name, stats, flush=True)
