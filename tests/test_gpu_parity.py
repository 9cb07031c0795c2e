"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerance for floating-point results (the GEMM): element-wise
|gpu - ref| <= 2e-2 |ref| + 1e-3 and relL2 < 3e-3 against the bf16-rounded
oracle, the relL2 gate being the one mori PR 785 (section Test) and PR 809
(section Results) validate against.  Exact-arithmetic inputs (small integer
codes, power-of-two scales) must match bitwise, as must the quantisers'
codes and scales.  Each case is printed before it runs, so a failure names
its shape and seed.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from dense_matmul_amd import inputs
from oracle import tolerance

pytestmark = pytest.mark.gpu

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
REL_L2 = GOLD["rel_l2_gate"]["value"]
DEV = "cuda:0"


@pytest.fixture(scope="module")
def dmm():
    import dense_matmul_amd as d

    d.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return d


def announce(*a):
    print("[case]", *a, flush=True)


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_close(got_bits, ref_bits, what, mode=None, operands=None, rows=None):
    """The acceptance rule of oracle.tolerance (the element-wise gate
    |err| <= 2e-2 |ref| + 1e-3 and relL2 < 3e-3, plus the measured
    matrix-core bound for the rare near-zero outputs); prints the
    statistics."""
    stats = tolerance.check(got_bits, ref_bits, what, mode=mode, operands=operands, rows=rows)
    print("[stats]", what, stats, flush=True)
    return stats


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# ------------------------------------------------------------ quantisers
# row lengths on both sides of each kernel boundary (one wave per row up to
# 512 columns, two up to 2048 and 4096, four up to 7168, two passes beyond),
# with ragged last 64-chunk slices
@pytest.mark.parametrize("rows,cols,seed", [(512, 256, 1), (300, 1792, 2), (7, 7168, 3), (64, 16, 4),
                                           (33, 4096, 14), (3, 2064, 16), (5, 9216, 15), (9, 512, 17),
                                           (9, 528, 18), (11, 1040, 19), (6, 2048, 20), (6, 4112, 26),
                                           (5, 6160, 27), (4, 7184, 28)])
def test_quantize_per_token_bitexact(dmm, rows, cols, seed):
    announce("quantize_per_token", rows, cols, seed)
    x = inputs.normal((rows, cols), seed)
    x[0] = 0.0
    if rows > 2:
        x[1] = 0.0
        x[1, cols // 2] = -3.25
        x[2] *= 1e-3
    q, s = dmm.quantize_per_token(to_dev(x))
    oq, os_ = oracle.quantize_per_token(x)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("rows,cols,seed", [(512, 256, 21), (300, 1792, 22), (5, 7168, 23), (33, 4096, 24),
                                           (5, 9216, 25), (7, 528, 29), (6, 4112, 30)])
def test_quantize_per_token_bf16_input_bitexact(dmm, rows, cols, seed):
    """bf16 activations: the oracle quantises the same values widened to fp32
    (bf16 -> fp32 is exact), so codes and scales must match bitwise."""
    announce("quantize_per_token bf16", rows, cols, seed)
    x = torch.from_numpy(inputs.normal((rows, cols), seed)).to(torch.bfloat16)  # RNE on the CPU
    x[0] = 0.0
    x[1, 3] = 448.0 * 3.0
    q, s = dmm.quantize_per_token(x.to(DEV))
    oq, os_ = oracle.quantize_per_token(x.to(torch.float32).numpy())
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("m,k,seed", [(300, 384, 5), (64, 128, 6), (33, 2048, 7)])
def test_quantize_blockscale_a_bitexact(dmm, m, k, seed):
    announce("quantize_blockscale_a", m, k, seed)
    x = inputs.normal((m, k), seed)
    x[3, 128:256] = 0.0
    q, s = dmm.quantize_blockscale_a(to_dev(x))
    oq, os_ = oracle.quantize_blockscale_a(x)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy(), os_)


@pytest.mark.parametrize("n,k,seed", [(272, 384, 8), (16, 128, 9), (1168, 256, 10)])
def test_quantize_blockscale_b_bitexact(dmm, n, k, seed):
    announce("quantize_blockscale_b", n, k, seed)
    x = inputs.normal((n, k), seed)
    q, s = dmm.quantize_blockscale_b(to_dev(x))
    oq, os_ = oracle.quantize_blockscale_b(x)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy(), os_)


@pytest.mark.parametrize("rows,k,seed", [(300, 384, 11), (17, 1792, 12), (64, 128, 13)])
def test_quantize_mxfp8_bitexact(dmm, rows, k, seed):
    announce("quantize_mxfp8", rows, k, seed)
    x = inputs.normal((rows, k), seed)
    x[1, 32:64] = 0.0
    x[2, :32] *= 1e-20
    x[3, 64:96] *= 1e4
    q, e = dmm.quantize_mxfp8(to_dev(x))
    oq, oe = oracle.quantize_mxfp8(x)
    assert np.array_equal(e.cpu().numpy(), oe)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq)


def e4m3_grid():
    """The non-negative finite E4M3 values in increasing order: 7 subnormal
    steps of 2^-9, then (1 + f/8) 2^(e-7) for exponent fields 1..15 (the
    all-ones fraction of field 15 is NaN)."""
    vals = [c / 512.0 for c in range(8)]
    vals += [(1 + f / 8.0) * 2.0 ** (e - 7) for e in range(1, 16) for f in range(8) if not (e == 15 and f == 7)]
    return np.array(vals)


def nudged(values, ulps):
    """float32 values moved by each of ``ulps`` units in the last place
    (values > 0, so a step of the bit pattern is a step of one ulp)."""
    b = np.asarray(values, np.float32).view(np.int32)
    return np.concatenate([(b + u).view(np.float32) for u in ulps])


def midpoint_matrix(rows_per_scale, k, group, amax_of, scales, seed):
    """Rows in bands of ``rows_per_scale``, band i quantised under scale
    ``scales[i]``: every ``group`` values along a row start with the group's
    maximum amax_of(scale) (so the group's scale is the band's) and the rest
    are drawn from values whose quotient by that scale lands within 6 ulps
    of an E4M3 rounding midpoint or grid point, with either sign, plus zeros
    and values under 2^-6 of the scale."""
    grid = e4m3_grid()
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(seed)
    x = np.empty((rows_per_scale * len(scales), k), np.float32)
    for i, sc in enumerate(scales):
        pool = nudged(np.concatenate([mids, grid[1:]]) * sc, range(-6, 7))
        pool = np.concatenate([pool, np.float32(sc) * np.array([0.0, 2.0 ** -7, 2.0 ** -11, 1e-3], np.float32)])
        band = rng.choice(pool, size=(rows_per_scale, k)) * rng.choice(np.array([-1, 1], np.float32), (rows_per_scale, k))
        band[:, ::group] = np.float32(amax_of(sc))
        x[i * rows_per_scale:(i + 1) * rows_per_scale] = band
    return x


# scales of no special form, a power of two, one near the top of the fp32
# range (maximum 2.7e38), and a subnormal one (the scale of a group whose
# maximum is 1e-38 is below 2^-126)
DIV_SCALES = [1.3, 0.0071, 97.31, 2.0, 3.0e-30, 6.0e35, 1e-38 / 448]


def test_quantizers_near_rounding_midpoints_bitexact(dmm):
    """Quotients within a few ulps of E4M3 rounding midpoints: the GPU
    quantisers encode v / s through a product with the reciprocal and the
    hardware converter, and fall back to the division only near midpoints,
    so these are the values where a wrong window or a wrong rounding would
    show.  Codes and scales must match the oracle bitwise."""
    x = midpoint_matrix(128, 3328, 128, lambda sc: np.float32(448.0 * sc), DIV_SCALES, 31)
    announce("quantizers near midpoints", x.shape)
    for name in ("quantize_per_token", "quantize_blockscale_a", "quantize_blockscale_b"):
        q, s = getattr(dmm, name)(to_dev(x))
        oq, os_ = getattr(oracle, name)(x)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), name
        got = q.view(torch.uint8).cpu().numpy()
        bad = np.argwhere(got != oq)
        assert bad.size == 0, (name, len(bad), [(int(r), int(c), float(x[r, c]), int(got[r, c]), int(oq[r, c]))
                                                 for r, c in bad[:5]])
    # bf16 input: the same values rounded to bf16 (a coarser set, still near midpoints)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    q, s = dmm.quantize_per_token(xb.to(DEV))
    oq, os_ = oracle.quantize_per_token(xb.to(torch.float32).numpy())
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def test_quantize_direct_range_exhaustive(dmm):
    """Every fp32 value of magnitude in [2^-6, 448], both signs (247.5 M
    values), quantised per token under a scale of exactly 1 (each row starts
    with 448): the quotient is the value itself, so this runs the GPU
    encoder's direct path (the hardware E4M3 conversion) over its whole input
    range, and the division path at every midpoint window, against the
    oracle's encoder, bitwise."""
    lo, hi = 0x3C800000, 0x43E00000  # 2^-6 and 448
    mags = np.arange(lo, hi + 1, dtype=np.uint32)
    vals = np.concatenate([mags, mags | np.uint32(0x80000000)]).view(np.float32)
    cols = (1 << 20) + 16
    per_row = cols - 1
    rows = -(-vals.size // per_row)
    body = np.full(rows * per_row, np.float32(1.0))
    body[: vals.size] = vals
    x = np.empty((rows, cols), np.float32)
    x[:, 0] = np.float32(448.0)
    x[:, 1:] = body.reshape(rows, per_row)
    assert np.array_equal(x[:, 1:].reshape(-1)[: vals.size].view(np.uint32), vals.view(np.uint32))
    announce("quantize_per_token exhaustive direct range", x.shape)
    del mags, vals, body
    q, s = dmm.quantize_per_token(to_dev(x))
    assert (s.cpu().numpy() == 1.0).all()
    got = q.view(torch.uint8).cpu().numpy()
    oq, os_ = oracle.quantize_per_token(x)
    assert (os_ == 1.0).all()
    bad = np.argwhere(got != oq)
    assert bad.size == 0, (len(bad), [(float(x[r, c]), int(got[r, c]), int(oq[r, c])) for r, c in bad[:5]])


def test_quantize_mxfp8_direct_range_exhaustive(dmm):
    """mxfp8 scales by 2^0 when a group's maximum is 448, so every other
    value of the group reaches the hardware E4M3 conversion unchanged: every
    fp32 value of magnitude in [2^-10, 448] (the E4M3 subnormal steps
    included), both signs, plus every 4096th pattern below 2^-10 (fp32
    subnormals included), against the oracle's encoder, bitwise."""
    lo, hi = 0x3A800000, 0x43E00000  # 2^-10 and 448
    mags = np.concatenate([np.arange(0, lo, 4096, dtype=np.uint32), np.arange(lo, hi + 1, dtype=np.uint32)])
    vals = np.concatenate([mags, mags | np.uint32(0x80000000)]).view(np.float32)
    k = 1 << 20
    groups = -(-vals.size // 31)
    body = np.full(groups * 31, np.float32(1.0))
    body[: vals.size] = vals
    g = np.empty((groups, 32), np.float32)
    g[:, 0] = np.float32(448.0)
    g[:, 1:] = body.reshape(groups, 31)
    rows = -(-groups // (k // 32))
    x = np.full((rows * (k // 32), 32), np.float32(448.0))
    x[:groups] = g
    x = x.reshape(rows, k)
    announce("quantize_mxfp8 exhaustive direct range", x.shape)
    del mags, vals, body, g
    q, e = dmm.quantize_mxfp8(to_dev(x))
    oq, oe = oracle.quantize_mxfp8(x)
    assert (oe == 127).all() and np.array_equal(e.cpu().numpy(), oe)
    got = q.view(torch.uint8).cpu().numpy()
    bad = np.argwhere(got != oq)
    assert bad.size == 0, (len(bad), [(float(x[r, c]), int(got[r, c]), int(oq[r, c])) for r, c in bad[:5]])


def test_quantizers_non_finite_inputs_bitexact(dmm):
    """NaN and infinities in the input: every quantiser's maximum ignores
    NaN (fmax), an infinite maximum gives an infinite fp32 scale (finite
    values quantise to zero, infinities to NaN) or the largest E8M0
    exponent; codes and scales match the oracle bitwise."""
    rng = np.random.default_rng(77)
    x = rng.standard_normal((256, 512)).astype(np.float32)
    for r in range(0, 256, 3):
        x[r, rng.integers(0, 512)] = np.nan
    for r in range(1, 256, 5):
        x[r, rng.integers(0, 512)] = np.inf
    for r in range(2, 256, 7):
        x[r, rng.integers(0, 512)] = -np.inf
    x[4, 0:128] = np.nan  # a whole row block of NaN in one 128-wide block
    x[5, 32:64] = 0.0
    x[5, 40] = np.nan  # a group whose maximum is 0
    announce("quantizers non-finite inputs", x.shape)
    for name in ("quantize_per_token", "quantize_blockscale_a", "quantize_blockscale_b"):
        q, s = getattr(dmm, name)(to_dev(x))
        oq, os_ = getattr(oracle, name)(x)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), name
        assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq), name
    q, e = dmm.quantize_mxfp8(to_dev(x))
    oq, oe = oracle.quantize_mxfp8(x)
    assert np.array_equal(e.cpu().numpy(), oe)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq)


def test_quantize_mxfp8_near_rounding_midpoints_bitexact(dmm):
    """mxfp8 scales by a power of two exactly, so values at E4M3 midpoints
    times the group's power of two are exact ties (round to even) and their
    ulp neighbours fall either side; the hardware converter must encode them
    as the oracle does."""
    x = midpoint_matrix(32, 3328, 32, lambda sc: np.float32(448.0 * sc), [2.0 ** -3, 2.0 ** 5, 2.0 ** -60, 2.0 ** 118], 32)
    announce("quantize_mxfp8 near midpoints", x.shape)
    q, e = dmm.quantize_mxfp8(to_dev(x))
    oq, oe = oracle.quantize_mxfp8(x)
    assert np.array_equal(e.cpu().numpy(), oe)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), oq)


# ------------------------------------------------------------ preshuffle
def documented_src_row(j, r, n):
    """B row held by fragment row r of block j, as include/dmm.h and
    preshuffle_b document it: blocks come in groups of four (64 output
    columns); in a group of p blocks, a block with a partner puts row r at
    column 32 (nb // 2) + 8 (r // 4) + 4 (nb % 2) + r % 4 of the group, the
    lone last block of an odd group keeps row order (16 nb + r)."""
    G, nb = divmod(j, 4)
    p = min(4, n // 16 - 4 * G)
    if p % 2 == 1 and nb == p - 1:
        return 64 * G + 16 * nb + r
    return 64 * G + 32 * (nb // 2) + 8 * (r // 4) + 4 * (nb % 2) + r % 4


def unshuffle(bs, n, k):
    """Inverse of the library's B order, written from its documented layout:
    chunk (j, kt) of 2 KiB; byte 16 l + t of half h is
    B[src(j, l % 16)][128 kt + 64 h + 16 (l / 16) + t]."""
    ki = k // 128
    v = bs.reshape(n // 16, ki, 2, 4, 16, 16)  # j, kt, h, l/16 (g), l%16 (r), t
    frag = v.transpose(0, 4, 1, 2, 3, 5).reshape(n // 16, 16, k)  # [j][r] = row data in fragment order
    out = np.empty((n, k), np.uint8)
    for j in range(n // 16):
        for r in range(16):
            out[documented_src_row(j, r, n)] = frag[j, r]
    return out


@pytest.mark.parametrize("n,k", [(16, 128), (32, 128), (48, 256), (272, 384), (1120, 256), (1168, 1792), (6288, 128)])
def test_preshuffle_is_the_documented_permutation(dmm, n, k):
    announce("preshuffle_b", n, k)
    b = np.random.default_rng(n + k).integers(0, 256, size=(n, k), dtype=np.uint8)
    bs = dmm.preshuffle_b(to_dev(b)).cpu().numpy()
    assert np.array_equal(np.bincount(bs.ravel(), minlength=256), np.bincount(b.ravel(), minlength=256))
    assert np.array_equal(unshuffle(bs, n, k), b)


# ------------------------------------------------------------------ GEMM
# ptpc runs on two tile shapes; "ptpc" is the library's own choice, the
# other two force one shape (same data, same oracle).
PTPC_TILE = {"ptpc": "auto", "ptpc_w": "256x256", "ptpc_n": "128x256", "ptpc_q": "128x128"}
# mxfp8 likewise: "mxfp8" forces the 256x256 tile, "mxfp8_n" the 256x128 one
MXFP8_TILE = {"mxfp8": "256x256", "mxfp8_n": "256x128", "mxfp8_auto": "auto"}
# blockscale: "blockscale" forces the 128x256 tile, "blockscale_n" the 128x128 one
BLOCKSCALE_TILE = {"blockscale": "128x256", "blockscale_n": "128x128", "blockscale_auto": "auto"}
MODE_ID = {"ptpc": 0, "blockscale": 1, "mxfp8": 2}
GEMM_MODES = ["ptpc_w", "ptpc_n", "ptpc_q", "blockscale", "blockscale_n", "mxfp8", "mxfp8_n"]


def base_mode(mode):
    return "ptpc" if mode in PTPC_TILE else "mxfp8" if mode in MXFP8_TILE else "blockscale"


def gemm_fn(dmm, mode):
    if mode in PTPC_TILE:
        return lambda *args, **kw: dmm.gemm_a8w8_ptpc(*args, tile=PTPC_TILE[mode], **kw)
    if mode in MXFP8_TILE:
        return lambda *args, **kw: dmm.gemm_a8w8_mxfp8(*args, tile=MXFP8_TILE[mode], **kw)
    return lambda *args, **kw: dmm.gemm_a8w8_blockscale(*args, tile=BLOCKSCALE_TILE[mode], **kw)


def tile_rows(mode):
    return 128 if mode in ("blockscale", "blockscale_n", "ptpc_n", "ptpc_q") else 256


def quantised_operands(mode, m, n, k, seed_a, seed_b):
    """fp32 N(0,1) operands quantised by the oracle's quantisers."""
    mode = base_mode(mode)
    a = inputs.operand_a(m, k, seed_a)
    b = inputs.normal((n, k), seed_b)
    if mode == "ptpc":
        qa, sa = oracle.quantize_per_token(a)
        qb, sb = oracle.quantize_per_token(b)
    elif mode == "blockscale":
        qa, sa = oracle.quantize_blockscale_a(a)
        qb, sb = oracle.quantize_blockscale_b(b)
    else:
        qa, sa = oracle.quantize_mxfp8(a)
        qb, sb = oracle.quantize_mxfp8(b)
    return qa, qb, sa, sb


def gpu_gemm(dmm, mode, qa, qb, sa, sb, out=None):
    b_shuf = dmm.preshuffle_b(to_dev(qb))
    return gemm_fn(dmm, mode)(to_dev(qa), b_shuf, to_dev(sa), to_dev(sb), out=out)


def exact_operands(mode, m, n, k, seed):
    mode = base_mode(mode)
    vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0], np.float32)
    codes = oracle.enc_e4m3(vals)
    qa = inputs.choice((m, k), codes, seed)
    qb = inputs.choice((n, k), codes, seed + 1)
    p2 = np.array([0.25, 0.5, 1.0, 2.0, 4.0], np.float32)
    if mode == "ptpc":
        sa, sb = inputs.choice((m,), p2, seed + 2), inputs.choice((n,), p2, seed + 3)
    elif mode == "blockscale":
        sa = inputs.choice((k // 128, m), p2, seed + 2)
        sb = inputs.choice(((n + 127) // 128, k // 128), p2, seed + 3)
    else:
        e = np.arange(125, 130, dtype=np.uint8)
        sa, sb = inputs.choice((k // 32, m), e, seed + 2), inputs.choice((k // 32, n), e, seed + 3)
    return qa, qb, sa, sb


# N % 64 = 16, 16, 16, 0, 16, 48, 32, 32: every kind of last column group
# K = 4096 takes the other C store policy of the 256-wide tiles
EXACT_SHAPES = [(1, 16, 128), (17, 272, 256), (300, 1168, 384), (256, 256, 512), (513, 528, 640), (64, 48, 1792),
                (130, 1120, 256), (40, 32, 128), (260, 272, 4096)]


@pytest.mark.parametrize("mode", GEMM_MODES)
@pytest.mark.parametrize("m,n,k", EXACT_SHAPES)
def test_gemm_exact_regime_bitwise(dmm, mode, m, n, k):
    """Every partial sum exact in fp32: the GPU must equal the oracle bitwise,
    including the partial last row and column tiles and K = 128 / 256."""
    announce("exact", mode, m, n, k)
    qa, qb, sa, sb = exact_operands(mode, m, n, k, m + n + k)
    c = gpu_gemm(dmm, mode, qa, qb, sa, sb)
    ref = oracle.gemm_a8w8(MODE_ID[base_mode(mode)], qa, qb, sa, sb)
    got = bf16_bits(c)
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{mode} {m}x{n}x{k}: {len(mism)} mismatches, first at {mism[:4].tolist()}"


@pytest.mark.parametrize("mode", GEMM_MODES)
@pytest.mark.parametrize("m,n,k,sa_seed,sb_seed", [(512, 1024, 256, 1, 2), (300, 1168, 1792, 61, 62),
                                                   (17, 16, 128, 3, 4), (1000, 3648, 512, 5, 6)])
def test_gemm_normal_inputs_within_tolerance(dmm, mode, m, n, k, sa_seed, sb_seed):
    announce("normal", mode, m, n, k)
    qa, qb, sa, sb = quantised_operands(mode, m, n, k, sa_seed, sb_seed)
    c = gpu_gemm(dmm, mode, qa, qb, sa, sb)
    ref = oracle.gemm_a8w8(MODE_ID[base_mode(mode)], qa, qb, sa, sb)
    check_close(bf16_bits(c), ref, f"{mode} {m}x{n}x{k}", base_mode(mode), (qa, qb, sa, sb))


def run_poisoned(dmm, mode, qa, qb, sa, sb, launches, hog=False):
    """``launches`` launches, each into a freshly NaN-poisoned C followed by a
    4 KiB canary; returns the outputs (bf16 bits) of every launch."""
    m, n = qa.shape[0], qb.shape[0]
    b_shuf = dmm.preshuffle_b(to_dev(qb))
    a, s_a, s_b = to_dev(qa), to_dev(sa), to_dev(sb)
    fn = gemm_fn(dmm, mode)
    buf = torch.empty(m * n + 2048, dtype=torch.bfloat16, device=DEV)
    c = buf[: m * n].view(m, n)
    canary = buf[m * n:]
    hog_src = torch.empty(64 << 20, dtype=torch.uint8, device=DEV) if hog else None
    hog_dst = torch.empty_like(hog_src) if hog else None
    side = torch.cuda.Stream() if hog else None
    outs = []
    for _ in range(launches):
        buf.fill_(float("nan"))
        canary.view(torch.int16).fill_(0x5A5A)
        if hog:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(4):
                    hog_dst.copy_(hog_src)
        fn(a, b_shuf, s_a, s_b, out=c)
        torch.cuda.synchronize()
        assert (canary.view(torch.int16) == 0x5A5A).all(), "write past the end of C"
        outs.append(bf16_bits(c))
    return outs


@pytest.mark.parametrize("mode", ["ptpc", "ptpc_w", "ptpc_n", "ptpc_q", "mxfp8", "mxfp8_n", "blockscale", "blockscale_n"])
@pytest.mark.parametrize("m,n,k,seed_a,seed_b", [(4096, 7168, 256, 11, 12), (16384, 7168, 512, 21, 22)])
def test_race_shapes_bit_stable_and_correct(dmm, mode, m, n, k, seed_a, seed_b):
    """The pages' race shapes (mori PR 785, Test table), in every mode and
    tile shape: 20 launches into a NaN-poisoned C must be bitwise identical,
    leave no NaN, and match the oracle on sampled rows (every row of the
    first and last 256-row tiles plus one per 64-row band)."""
    announce("race", mode, m, n, k)
    qa, qb, sa, sb = quantised_operands(mode, m, n, k, seed_a, seed_b)
    outs = run_poisoned(dmm, mode, qa, qb, sa, sb, 20)
    for i, o in enumerate(outs[1:], 1):
        diff = np.count_nonzero(o != outs[0])
        assert diff == 0, f"launch {i} differs from launch 0 in {diff} elements"
    assert not np.isnan(bits_to_f64(outs[0])).any()
    rows = inputs.rows_sample(m, seed=m)
    ref = oracle.gemm_a8w8(MODE_ID[base_mode(mode)], qa, qb, sa, sb, rows=rows)
    check_close(outs[0][rows], ref, f"{mode} {m}x{n}x{k} sampled rows", base_mode(mode), (qa, qb, sa, sb), rows)


@pytest.mark.parametrize("mode", ["ptpc_w", "ptpc_n", "ptpc_q", "mxfp8", "mxfp8_n", "blockscale", "blockscale_n"])
def test_bit_stable_under_concurrent_copy(dmm, mode):
    """Same 20-launch identity with an HBM copy loop on a second stream."""
    m, n, k = 4096, 7168, 256
    announce("hog", mode, m, n, k)
    qa, qb, sa, sb = quantised_operands(mode, m, n, k, 11, 12)
    outs = run_poisoned(dmm, mode, qa, qb, sa, sb, 20, hog=True)
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(o, outs[0]), f"launch {i} differs"
    assert not np.isnan(bits_to_f64(outs[0])).any()


@pytest.mark.parametrize("tile", ["auto", "128x128", "64x64"])
def test_bf16_gemm(dmm, tile):
    m, k, n = GOLD["bf16_shape_mkn"]["value"]
    announce("bf16", m, k, n, tile)
    a32, b_kn = inputs.bf16_operands(m, k, n, GOLD["bf16_seed"]["value"])
    a = torch.from_numpy(a32).to(torch.bfloat16)
    b = torch.from_numpy(np.ascontiguousarray(b_kn.T)).to(torch.bfloat16)  # [N, K]
    ad, bd = a.to(DEV), b.to(DEV)
    # 20 launches, each into a freshly NaN-poisoned C followed by a canary
    # (DeepGEMM PR 453, Reproduction and validation: repeated launches of this
    # shape compared bit for bit)
    buf = torch.empty(m * n + 2048, dtype=torch.bfloat16, device=DEV)
    c = buf[: m * n].view(m, n)
    canary = buf[m * n:].view(torch.int16)
    first = None
    for i in range(20):
        buf.fill_(float("nan"))
        canary.fill_(0x5A5A)
        dmm.gemm_bf16(ad, bd, out=c, tile=tile)
        if first is None:
            first = c.clone()
            assert not torch.isnan(first).any().item(), "unwritten elements"
        else:
            assert torch.equal(c.view(torch.int16), first.view(torch.int16)), f"launch {i} differs from launch 0"
        assert bool((canary == 0x5A5A).all().item()), f"launch {i} wrote past the end of C"
    ref = oracle.gemm_bf16(a.view(torch.int16).numpy().view(np.uint16), b.view(torch.int16).numpy().view(np.uint16))
    check_close(bf16_bits(first), ref, f"bf16 4096x1024x896 {tile}")


@pytest.mark.parametrize("tile", ["128x128", "64x64"])
@pytest.mark.parametrize("m,n,k", [(1, 16, 64), (200, 272, 192), (129, 144, 1024), (300, 1040, 320)])
def test_bf16_gemm_edges(dmm, m, n, k, tile):
    """Exact inputs (small integers and halves, sums far below 2^24): bitwise
    equal to the oracle on both tile shapes, with partial row and column
    tiles and K tile counts that end mid-way through the 3-stage ring."""
    announce("bf16 edge", m, n, k, tile)
    vals = np.array([0, 1, -1, 2, -2, 0.5], np.float32)
    a = torch.from_numpy(inputs.choice((m, k), vals, m)).to(torch.bfloat16)
    b = torch.from_numpy(inputs.choice((n, k), vals, n)).to(torch.bfloat16)
    c = dmm.gemm_bf16(a.to(DEV), b.to(DEV), tile=tile)
    ref = oracle.gemm_bf16(a.view(torch.int16).numpy().view(np.uint16), b.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(bf16_bits(c), ref)


def test_invalid_arguments_raise_value_error(dmm):
    a = torch.zeros((64, 256), dtype=torch.uint8, device=DEV)
    b = torch.zeros((24, 256), dtype=torch.uint8, device=DEV)  # N not a multiple of 16
    s = torch.ones(64, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        dmm.gemm_a8w8_ptpc(a, b, s, torch.ones(24, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        dmm.gemm_a8w8_ptpc(a[:, :200].contiguous(), b[:16, :200].contiguous(), s,
                           torch.ones(16, dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("mode", ["ptpc_w", "ptpc_n", "ptpc_q", "mxfp8", "mxfp8_n", "blockscale", "blockscale_n"])
@pytest.mark.parametrize("k", [128, 256, 384, 512, 640])
def test_many_tiles_per_workgroup_every_k_phase(dmm, mode, k):
    """More tiles than CUs, so every workgroup runs 2-3 tiles back to back,
    for each K / 128 mod 4: the stage phase of a tile's first K tile cycles
    through 1, 2 or 4 values and (ptpc, mxfp8) each tile's epilogue runs in
    the next tile's first K step.  Exact-arithmetic inputs: sampled rows of
    every tile row band must equal the oracle bitwise; two launches into a
    NaN-poisoned C must be identical and leave no NaN."""
    bm = tile_rows(mode)
    m, n = 18 * bm + 40, 8192 + 48  # partial last row and column tiles
    announce("many tiles", mode, m, n, k)
    qa, qb, sa, sb = exact_operands(mode, m, n, k, 7 * k + len(mode))
    outs = run_poisoned(dmm, mode, qa, qb, sa, sb, 2)
    diff = np.count_nonzero(outs[1] != outs[0])
    assert diff == 0, f"launch 1 differs from launch 0 in {diff} elements"
    assert not np.isnan(bits_to_f64(outs[0])).any(), "rows or columns left unwritten"
    rows = np.unique(np.clip(np.concatenate([t * bm + np.array([0, 1, 15, 16, bm - 1]) for t in range(19)]), 0, m - 1))
    ref = oracle.gemm_a8w8(MODE_ID[base_mode(mode)], qa, qb, sa, sb, rows=rows)
    got = outs[0][rows]
    mism = np.argwhere(got != ref)
    assert mism.size == 0, f"{mode} {m}x{n}x{k}: {len(mism)} mismatches, first at {mism[:4].tolist()}"
