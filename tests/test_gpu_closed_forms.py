"""GPU closed forms: the HIP GEMM, through the C ABI, against results that
the definition

    C[m, n] = bf16( sum_k (A[m, k] sa(m, k)) (B[n, k] sb(n, k)) ),  fp32 accumulation

(mori PR 785, "fix(gemm-ar): drain the peeled tail's producers instead of
tightening the loop", Cost: the ptpc, blockscale and mxfp8 modes) fixes
without any oracle:

- identity B (N = K, codes 1.0, unit B scales): C = bf16(dec(A) sa),
  element by element;
- a one-hot B (row n holds 1.0 at column p(n), p injective):
  C[:, n] = bf16(dec(A[:, p(n)]) sa(:, p(n)));
- A = 0: C = 0;
- A made only of subnormal E4M3 codes, identity B: the same exact closed
  form, so the matrix core keeps fp8 subnormals;
- doubling every A scale (the E8M0 byte + 1 for mxfp8) doubles C exactly:
  a power-of-two factor commutes with every fp32 and bf16 rounding at these
  magnitudes;
- mxfp8 with every scale byte 127 (2^0) is ptpc with unit scales, and the
  two ptpc tile shapes compute the same sums in the same order: the same
  codes give the same bits.

In each closed form the sum has a single non-zero term (or none), so it is
exact in any order; decoding uses torch's CPU float8_e4m3fn cast and
rounding torch's CPU bfloat16 cast (library routines).  Zeros compare by
value: where the selected code is -0 the other terms are zeros of either
sign, and an fp32 sum of mixed-sign zeros is +0.  The shapes include
a partial last row tile (M = 300), a partial last 256-column tile and K
with a main loop and a peeled tail.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_matmul_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ONE = 0x38  # E4M3 code of 1.0
MODES = ["ptpc_w", "ptpc_n", "ptpc_q", "blockscale", "blockscale_n", "mxfp8", "mxfp8_n"]


@pytest.fixture(scope="module")
def dmm():
    import dense_matmul_amd as d

    d.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return d


def announce(*a):
    print("[case]", *a, flush=True)


def dec(codes):
    """E4M3 codes -> fp32 values (torch's CPU cast)."""
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def bf16_bits_of(f32):
    """fp32 -> bf16 bit patterns, round to nearest even (torch's CPU cast)."""
    return torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def zero_as_plus(bits):
    """bf16 bits with -0 read as +0 (zeros compare by value)."""
    return np.where(bits == 0x8000, np.uint16(0), bits)


def run(dmm, mode, qa, qb, sa, sb):
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    b_shuf = dmm.preshuffle_b(dev(qb))
    a, s_a, s_b = dev(qa), dev(sa), dev(sb)
    if mode in ("ptpc_w", "ptpc_n", "ptpc_q"):
        c = dmm.gemm_a8w8_ptpc(a, b_shuf, s_a, s_b, tile={"ptpc_w": "256x256", "ptpc_n": "128x256", "ptpc_q": "128x128"}[mode])
    elif mode.startswith("blockscale"):
        c = dmm.gemm_a8w8_blockscale(a, b_shuf, s_a, s_b, tile={"blockscale": "128x256", "blockscale_n": "128x128"}[mode])
    else:
        c = dmm.gemm_a8w8_mxfp8(a, b_shuf, s_a, s_b, tile={"mxfp8": "256x256", "mxfp8_n": "256x128"}[mode])
    torch.cuda.synchronize()
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


def a_codes(m, k, seed):
    """E4M3 codes of N(0,1) data quantised per row (any finite codes do)."""
    return oracle.quantize_per_token(inputs.normal((m, k), seed))[0]


def a_scales(mode, m, k, seed):
    """Arbitrary A scales of the mode and sa(m, k) as an [m, k] fp32 array."""
    rng = np.random.default_rng(seed)
    if mode.startswith("mxfp8"):
        e = rng.integers(120, 135, size=(k // 32, m)).astype(np.uint8)
        full = np.ldexp(np.float32(1), e.astype(np.int32) - 127).astype(np.float32)  # exact powers of two
        return e, np.repeat(full.T, 32, axis=1)
    if mode.startswith("blockscale"):
        s = rng.uniform(0.5, 2.0, size=(k // 128, m)).astype(np.float32)
        return s, np.repeat(s.T, 128, axis=1)
    s = rng.uniform(0.5, 2.0, size=(m,)).astype(np.float32)
    return s, np.repeat(s[:, None], k, axis=1)


def unit_b_scales(mode, n, k):
    if mode.startswith("mxfp8"):
        return np.full((k // 32, n), 127, np.uint8)
    if mode.startswith("blockscale"):
        return np.ones(((n + 127) // 128, k // 128), np.float32)
    return np.ones((n,), np.float32)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("m,k", [(300, 384), (64, 256), (17, 128), (1, 128)])
def test_identity_b(dmm, mode, m, k):
    """B = I (N = K): C[m, n] = bf16(dec(A[m, n]) * sa(m, n)), bitwise."""
    announce("identity B", mode, m, k)
    qa = a_codes(m, k, 900 + k)
    sa, sa_full = a_scales(mode, m, k, 901 + m)
    qb = np.zeros((k, k), np.uint8)
    qb[np.arange(k), np.arange(k)] = ONE
    got = run(dmm, mode, qa, qb, sa, unit_b_scales(mode, k, k))
    want = bf16_bits_of(dec(qa) * sa_full)
    bad = np.argwhere(zero_as_plus(got) != zero_as_plus(want))
    assert bad.size == 0, f"{mode} {m}x{k}: {len(bad)} mismatches, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("m,n,k", [(300, 272, 640), (1, 16, 128), (513, 1168, 1792)])
def test_one_hot_b_selects_columns(dmm, mode, m, n, k):
    """Row n of B holds 1.0 at column p(n): C[:, n] = bf16(dec(A[:, p(n)]) sa(:, p(n)))."""
    announce("one-hot B", mode, m, n, k)
    qa = a_codes(m, k, 910 + m)
    sa, sa_full = a_scales(mode, m, k, 911 + n)
    p = np.random.default_rng(912 + k).permutation(k)[:n]
    qb = np.zeros((n, k), np.uint8)
    qb[np.arange(n), p] = ONE
    got = run(dmm, mode, qa, qb, sa, unit_b_scales(mode, n, k))
    want = bf16_bits_of(dec(qa)[:, p] * sa_full[:, p])
    bad = np.argwhere(zero_as_plus(got) != zero_as_plus(want))
    assert bad.size == 0, f"{mode}: {len(bad)} mismatches, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("mode", MODES)
def test_subnormal_codes_are_kept(dmm, mode):
    """A made only of the fourteen subnormal E4M3 codes (+-f 2^-9, f = 1..7),
    identity B: every output is bf16(dec(A) sa) exactly, so the matrix core
    neither flushes nor rescales fp8 subnormal inputs."""
    m, k = 300, 384
    announce("subnormal A", mode, m, k)
    subs = np.array([f | s for f in range(1, 8) for s in (0, 0x80)], np.uint8)
    qa = inputs.choice((m, k), subs, 950)
    sa, sa_full = a_scales(mode, m, k, 951)
    qb = np.zeros((k, k), np.uint8)
    qb[np.arange(k), np.arange(k)] = ONE
    got = run(dmm, mode, qa, qb, sa, unit_b_scales(mode, k, k))
    want = bf16_bits_of(dec(qa) * sa_full)
    assert np.all(dec(qa) != 0)
    bad = np.argwhere(zero_as_plus(got) != zero_as_plus(want))
    assert bad.size == 0, f"{mode}: {len(bad)} mismatches, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("mode", MODES)
def test_zero_a_gives_zero(dmm, mode):
    m, n, k = 300, 528, 512
    announce("zero A", mode, m, n, k)
    qb = a_codes(n, k, 920)
    sa, _ = a_scales(mode, m, k, 921)
    sb = unit_b_scales(mode, n, k)
    got = run(dmm, mode, np.zeros((m, k), np.uint8), qb, sa, sb)
    assert np.all((got & 0x7FFF) == 0), f"{mode}: non-zero outputs from A = 0"


@pytest.mark.parametrize("mode", MODES)
def test_doubling_a_scales_doubles_c(dmm, mode):
    """Every A scale times 2 (E8M0 byte + 1): every output bitwise 2x, on
    N(0,1) data where the sums are inexact."""
    m, n, k = 300, 1168, 1792
    announce("doubling", mode, m, n, k)
    base = "ptpc" if mode.startswith("ptpc") else "mxfp8" if mode.startswith("mxfp8") else "blockscale"
    a = inputs.normal((m, k), 930)
    b = inputs.normal((n, k), 931)
    quant = {"ptpc": (oracle.quantize_per_token, oracle.quantize_per_token),
             "blockscale": (oracle.quantize_blockscale_a, oracle.quantize_blockscale_b),
             "mxfp8": (oracle.quantize_mxfp8, oracle.quantize_mxfp8)}[base]
    qa, sa = quant[0](a)
    qb, sb = quant[1](b)
    sa2 = (sa + 1).astype(np.uint8) if base == "mxfp8" else (sa * 2).astype(np.float32)
    c1 = run(dmm, mode, qa, qb, sa, sb)
    c2 = run(dmm, mode, qa, qb, sa2, sb)
    to_f = lambda h: (h.astype(np.uint32) << 16).view(np.float32)
    assert np.isfinite(to_f(c1)).all()
    bad = np.argwhere(to_f(c2) != 2 * to_f(c1))
    assert bad.size == 0, f"{mode}: {len(bad)} outputs not doubled, first at {bad[:4].tolist()}"


def test_modes_agree_under_unit_scales(dmm):
    """mxfp8 with every scale 2^0, ptpc with unit scales on either tile shape:
    the same codes give the same bits (N(0,1) codes, inexact sums)."""
    m, n, k = 300, 1168, 1792
    announce("unit scales across modes", m, n, k)
    qa = a_codes(m, k, 940)
    qb = a_codes(n, k, 941)
    ptpc_w = run(dmm, "ptpc_w", qa, qb, np.ones(m, np.float32), np.ones(n, np.float32))
    ptpc_n = run(dmm, "ptpc_n", qa, qb, np.ones(m, np.float32), np.ones(n, np.float32))
    ptpc_q = run(dmm, "ptpc_q", qa, qb, np.ones(m, np.float32), np.ones(n, np.float32))
    mx = run(dmm, "mxfp8", qa, qb, np.full((k // 32, m), 127, np.uint8), np.full((k // 32, n), 127, np.uint8))
    assert np.array_equal(ptpc_w, ptpc_n), f"ptpc tiles differ at {np.argwhere(ptpc_w != ptpc_n)[:4].tolist()}"
    assert np.array_equal(ptpc_w, ptpc_q), f"ptpc tiles differ at {np.argwhere(ptpc_w != ptpc_q)[:4].tolist()}"
    assert np.array_equal(ptpc_w, mx), f"ptpc and mxfp8 differ at {np.argwhere(ptpc_w != mx)[:4].tolist()}"


@pytest.mark.parametrize("tile", ["auto", "128x128", "64x64"])
@pytest.mark.parametrize("m,n,k", [(300, 272, 640), (1, 16, 64), (4096, 896, 1024)])
def test_bf16_one_hot_b_selects_columns(dmm, tile, m, n, k):
    """bf16 GEMM (DeepGEMM PR 453, "Fix SM120 BF16 GEMM shared-memory reuse
    ordering", Reproduction and validation: the [4096, 1024] x [1024, 896]
    shape among others): row n of B holds 1.0 at column p(n), so
    C[:, n] = A[:, p(n)] bit for bit (zeros by value)."""
    announce("bf16 one-hot B", tile, m, n, k)
    a = torch.from_numpy(inputs.normal((m, k), 960 + m)).to(torch.bfloat16)
    p = np.random.default_rng(961 + k).permutation(k)[:n]
    b = torch.zeros((n, k), dtype=torch.bfloat16)
    b[torch.arange(n), torch.from_numpy(p)] = 1.0
    c = dmm.gemm_bf16(a.to(DEV), b.to(DEV), tile=tile)
    torch.cuda.synchronize()
    got = c.view(torch.int16).cpu().numpy().view(np.uint16)
    want = a.view(torch.int16).numpy().view(np.uint16)[:, p]
    bad = np.argwhere(zero_as_plus(got) != zero_as_plus(want))
    assert bad.size == 0, f"bf16 {tile} {m}x{n}x{k}: {len(bad)} mismatches, first at {bad[:4].tolist()}"
