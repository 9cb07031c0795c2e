"""The precision of gfx950's fp8 matrix instructions, observed through the
public GEMM: the pin behind the secondary acceptance rule of
oracle.tolerance (RHO).

Each output of a 16 x 16 x 128 GEMM with unit scales is one matrix
instruction's sum of 128 exact fp8 products.  The operands are built so that
two large products cancel exactly (+P and -P at two K positions shared by
every row) while the other 126 products are small and random: the exact sum
is then tiny next to the largest product P, and the bf16 output (whose own
rounding is at most 2^-9 of that tiny sum, below 2^-17 P) shows the
instruction's rounding directly.  Over 64 launches per mode (16384 outputs)
the largest |gpu - exact| / P must be

  * at most RHO = 2^-11 (the bound the secondary rule uses), and
  * above zero: the instruction does not sum exactly, which is why a
    near-cancelling output can miss the fixed 1e-3 floor of the primary rule
    at all.

The exact sums are float64 sums of decoded codes (exact: every product has at
most 8 significant bits and every partial sum fits in 53).  Nothing here
depends on the summation order inside the instruction.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LAUNCHES = 64


@pytest.fixture(scope="module")
def dmm():
    import dense_matmul_amd as d

    d.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return d


def small_codes(rng, shape):
    """Random e4m3 codes of magnitude 2^-6 .. 2^2 (normals), random signs."""
    mag = np.ldexp(1.0 + rng.integers(0, 8, size=shape) / 8.0, rng.integers(-6, 2, size=shape)).astype(np.float32)
    sign = np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0).astype(np.float32)
    return oracle.enc_e4m3(mag * sign)


def cancelling_operands(seed):
    """A [16, 128] and B [16, 128] codes: at K positions k0, k1 every row of A
    holds +big and every row of B holds +big / -big, so those two products
    cancel exactly; everything else is small."""
    rng = np.random.default_rng(seed)
    qa, qb = small_codes(rng, (16, 128)), small_codes(rng, (16, 128))
    k0, k1 = rng.choice(128, size=2, replace=False)
    big = float(rng.choice([256.0, 448.0, 320.0, 128.0]))
    qa[:, k0] = oracle.enc_e4m3(np.array([big], np.float32))[0]
    qa[:, k1] = oracle.enc_e4m3(np.array([big], np.float32))[0]
    sgn = 1.0 if rng.integers(0, 2) else -1.0
    qb[:, k0] = oracle.enc_e4m3(np.array([sgn * big], np.float32))[0]
    qb[:, k1] = oracle.enc_e4m3(np.array([-sgn * big], np.float32))[0]
    return qa, qb, big * big


def unit_scales(mode):
    if mode.startswith("ptpc"):
        return np.ones(16, np.float32), np.ones(16, np.float32)
    if mode == "blockscale":
        return np.ones((1, 16), np.float32), np.ones((1, 1), np.float32)
    return np.full((4, 16), 127, np.uint8), np.full((4, 16), 127, np.uint8)


def run(dmm, mode, qa, qb, sa, sb):
    t = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
    bs = dmm.preshuffle_b(t(qb))
    if mode == "ptpc":
        c = dmm.gemm_a8w8_ptpc(t(qa), bs, t(sa), t(sb))
    elif mode == "ptpc_w":
        c = dmm.gemm_a8w8_ptpc(t(qa), bs, t(sa), t(sb), tile="256x256")
    elif mode == "blockscale":
        c = dmm.gemm_a8w8_blockscale(t(qa), bs, t(sa), t(sb))
    else:
        c = dmm.gemm_a8w8_mxfp8(t(qa), bs, t(sa), t(sb))
    return tolerance.bits_to_f64(c.view(torch.int16).cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("mode", ["ptpc", "ptpc_w", "blockscale", "mxfp8"])
def test_one_instruction_rounds_within_rho_of_its_largest_product(dmm, mode):
    print("[case] matrix-core precision", mode, flush=True)
    worst, nonzero = 0.0, 0
    for s in range(LAUNCHES):
        qa, qb, pmax = cancelling_operands(1000 + s)
        sa, sb = unit_scales(mode)
        got = run(dmm, mode, qa, qb, sa, sb)
        exact = oracle.dec_e4m3(qa).astype(np.float64) @ oracle.dec_e4m3(qb).astype(np.float64).T
        assert np.abs(exact).max() < pmax * 2.0**-6, "the construction keeps the exact sums small"
        dev = np.abs(got - exact)
        # what the bf16 output rounding alone can explain
        out_round = np.ldexp(1.0, np.frexp(np.maximum(np.abs(exact), 1e-30))[1] - 9)
        nonzero += int(np.count_nonzero(dev > out_round))
        worst = max(worst, float(dev.max()) / pmax)
    print(f"[stats] {mode}: worst |gpu - exact| / max product = 2^{np.log2(max(worst, 1e-300)):.2f}; "
          f"{nonzero} of {LAUNCHES * 256} outputs beyond the bf16 output rounding", flush=True)
    assert worst <= tolerance.RHO, f"{mode}: instruction error {worst:.3g} of the largest product > RHO"
    assert nonzero > 0, f"{mode}: every sum exact -- the secondary rule's premise does not hold"
