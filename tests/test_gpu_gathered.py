"""GPU tests of the gathered-operand GEMM (gemm_a8w8_ptpc_gathered): the GEMM
half of an all-gather + GEMM on one GPU (mori PR 809, How it works: the
tile order and the wait).  The result must equal the plain ptpc GEMM
bitwise; a band's rows must not be read before its arrival flag reaches the
epoch (wrap-safe compare); a wait that never ends gives up after its spin
limit and reports the band, and the kernel still finishes."""
import time

import numpy as np
import pytest
import torch

import oracle
from dense_matmul_amd import inputs
from oracle import tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dmm():
    import dense_matmul_amd as d

    d.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return d


def announce(*a):
    print("[case]", *a, flush=True)


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def operands(m, n, k, nsrc):
    """A = nsrc stacked slabs, each from its own seed (the pages' gathered
    shapes stack 4096-row blocks of different ranks), quantised per token;
    B per channel."""
    qa, sa = oracle.quantize_per_token(inputs.operand_a(m, k, tuple(range(500, 500 + nsrc))))
    qb, sb = oracle.quantize_per_token(inputs.normal((n, k), 510))
    return qa, qb, sa, sb


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def as_i32(v):
    return int(np.array([v & 0xFFFFFFFF], np.uint32).view(np.int32)[0])


@pytest.mark.parametrize("own,nchunks,epoch,flag", [
    (2, 2, 5, 5),                       # flag == epoch
    (0, 4, 0xFFFFFFF0, 3),              # flag ahead of epoch across the 2^32 wrap
    (3, 1, 100, 100 + (1 << 30)),       # far ahead, still "reached"
])
def test_ready_bands_match_the_plain_gemm(dmm, own, nchunks, epoch, flag):
    m, n, k, nsrc = 4 * 1024, 1168, 512, 4
    announce("gathered ready", own, nchunks, hex(epoch), hex(flag))
    qa, qb, sa, sb = operands(m, n, k, nsrc)
    a, b_shuf, s_a, s_b = to_dev(qa), dmm.preshuffle_b(to_dev(qb)), to_dev(sa), to_dev(sb)
    plain = dmm.gemm_a8w8_ptpc(a, b_shuf, s_a, s_b, tile="256x256")
    flags = torch.full((nsrc * nchunks,), as_i32(flag), dtype=torch.int32, device=DEV)
    out = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    c, status = dmm.gemm_a8w8_ptpc_gathered(a, b_shuf, s_a, s_b, flags, m // nsrc, nchunks, own, epoch, out=out)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got, ref = bits(c), bits(plain)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} elements differ from gemm_a8w8_ptpc"
    rows = inputs.rows_sample(m, seed=7)
    tolerance.check(got[rows], oracle.gemm_ptpc(qa, qb, sa, sb, rows=rows), "gathered sampled rows", mode="ptpc",
                    operands=(qa, qb, sa, sb), rows=rows)


def test_waits_for_bands_written_after_launch(dmm):
    """Only the own slab is in A when the kernel starts; every other band is
    copied in from pinned host memory on a side stream after the launch and
    its flag (pinned host memory) set by this thread once the copy is done.
    The kernel must still be running before the first flag, and the result
    must be the plain GEMM's (the fence after each flag makes the new rows
    visible)."""
    m, n, k, nsrc, nchunks, own = 8 * 1024, 7168, 512, 8, 2, 5
    src_rows, band_rows = m // nsrc, m // nsrc // nchunks
    epoch = 0x7FFFFFFE
    announce("gathered late bands", m, n, k, nsrc, nchunks, own)
    qa, qb, sa, sb = operands(m, n, k, nsrc)
    b_shuf, s_b = dmm.preshuffle_b(to_dev(qb)), to_dev(sb)
    plain = dmm.gemm_a8w8_ptpc(to_dev(qa), b_shuf, to_dev(sa), s_b, tile="256x256")
    torch.cuda.synchronize()
    # device A and a_scale hold only the own slab; the rest is zero
    a = torch.zeros((m, k), dtype=torch.uint8, device=DEV)
    s_a = torch.zeros(m, dtype=torch.float32, device=DEV)
    lo, hi = own * src_rows, (own + 1) * src_rows
    a[lo:hi] = to_dev(qa[lo:hi])
    s_a[lo:hi] = to_dev(sa[lo:hi])
    host_a = torch.from_numpy(qa).pin_memory()
    host_s = torch.from_numpy(sa).pin_memory()
    flags = torch.full((nsrc * nchunks,), as_i32(epoch - 1), dtype=torch.int32).pin_memory()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    out, status = dmm.gemm_a8w8_ptpc_gathered(a, b_shuf, s_a, s_b, flags, src_rows, nchunks, own, epoch,
                                              spin_limit=1 << 19)
    t0 = time.time()
    time.sleep(0.05)
    still_running = not torch.cuda.current_stream().query()
    order = [((own + r) % nsrc, c) for c in range(nchunks) for r in range(1, nsrc)]
    for src, c in order:
        r0 = src * src_rows + c * band_rows
        with torch.cuda.stream(side):
            a[r0:r0 + band_rows].copy_(host_a[r0:r0 + band_rows], non_blocking=True)
            s_a[r0:r0 + band_rows].copy_(host_s[r0:r0 + band_rows], non_blocking=True)
        side.synchronize()
        flags[src * nchunks + c] = as_i32(epoch)
    torch.cuda.synchronize()
    elapsed = time.time() - t0
    assert still_running, "the kernel finished before any band had arrived"
    assert int(status.item()) == 0, "a wait gave up"
    got, ref = bits(out), bits(plain)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} elements differ ({elapsed:.3f} s)"


def test_a_wait_that_never_ends_gives_up(dmm):
    """No band but the own slab ever arrives: every wait gives up after its
    spin limit, status names the largest band, and the launch completes."""
    m, n, k, nsrc, nchunks, own = 4 * 512, 1168, 256, 4, 2, 1
    announce("gathered timeout")
    qa, qb, sa, sb = operands(m, n, k, nsrc)
    flags = torch.zeros(nsrc * nchunks, dtype=torch.int32, device=DEV)
    out, status = dmm.gemm_a8w8_ptpc_gathered(to_dev(qa), dmm.preshuffle_b(to_dev(qb)), to_dev(sa), to_dev(sb),
                                              flags, m // nsrc, nchunks, own, 1, spin_limit=50)
    torch.cuda.synchronize()
    want = max(s * nchunks + c for s in range(nsrc) for c in range(nchunks) if s != own) + 1
    assert int(status.item()) == want
