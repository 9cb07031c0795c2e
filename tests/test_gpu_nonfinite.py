"""GEMM operands holding E4M3 NaN codes (the format's two NaN patterns,
S.1111.111): the definition makes every output that sums a product with a NaN
operand NaN, so a NaN code in row m of A turns row m of C into NaN and one in
row n of B turns column n into NaN, whatever else the row holds.  Every mode
and tile, exact-regime data elsewhere (so the other outputs are bitwise), a
ragged M and every kind of last column group; NaN positions are compared
exactly (not NaN-bit patterns, which the definition does not fix), all other
outputs bitwise against the oracle."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import test_gpu_parity as par  # noqa: E402

pytestmark = pytest.mark.gpu
NAN_CODES = (0x7F, 0xFF)


@pytest.fixture(scope="module")
def dmm_nan():
    import dense_matmul_amd as d

    d.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return d


def test_nan_patterns_decode_to_nan():
    assert np.isnan(oracle.dec_e4m3(np.array(NAN_CODES, np.uint8))).all()


@pytest.mark.parametrize("mode", par.GEMM_MODES)
@pytest.mark.parametrize("m,n,k", [(300, 1168, 384), (513, 528, 640)])
def test_nan_codes_poison_exactly_their_rows_and_columns(dmm_nan, mode, m, n, k):
    par.announce("nan codes", mode, m, n, k)
    qa, qb, sa, sb = par.exact_operands(mode, m, n, k, seed=91)
    rng = np.random.default_rng(92)
    nan_rows, nan_cols = [0, 7, m - 1], [5, n - 1]
    for r in nan_rows:
        qa[r, rng.integers(0, k)] = NAN_CODES[r % 2]
    for c in nan_cols:
        qb[c, rng.integers(0, k)] = NAN_CODES[c % 2]
    got = par.bf16_bits(par.gpu_gemm(dmm_nan, mode, qa, qb, sa, sb))
    ref = oracle.gemm_a8w8(par.MODE_ID[par.base_mode(mode)], qa, qb, sa, sb)
    got_nan, ref_nan = np.isnan(par.bits_to_f64(got)), np.isnan(par.bits_to_f64(ref))
    want = np.zeros((m, n), bool)
    want[nan_rows, :] = True
    want[:, nan_cols] = True
    assert np.array_equal(ref_nan, want), "the oracle's NaN outputs are the poisoned rows and columns"
    assert np.array_equal(got_nan, want), f"{mode}: {np.count_nonzero(got_nan != want)} outputs differ in NaN-ness"
    assert np.array_equal(got[~want], ref[~want]), f"{mode}: {np.count_nonzero(got[~want] != ref[~want])} finite outputs differ"


@pytest.mark.parametrize("mode", par.GEMM_MODES)
def test_nan_scales_poison_exactly_their_rows_and_columns(dmm_nan, mode):
    """A NaN scale (fp32 NaN; for mxfp8 the E8M0 byte 255, NaN in OCP MX)
    makes every a' or b' it multiplies NaN: a row's scale poisons its row, a
    column's its column (blockscale: B's scale poisons its 128-column block)."""
    m, n, k = 300, 1168, 384
    par.announce("nan scales", mode, m, n, k)
    base = par.base_mode(mode)
    qa, qb, sa, sb = par.exact_operands(mode, m, n, k, seed=93)
    nan_rows, nan_cols = [3, m - 1], [9, n - 1]
    want = np.zeros((m, n), bool)
    want[nan_rows, :] = True
    if base == "ptpc":
        sa[nan_rows] = np.nan
        sb[nan_cols] = np.nan
        want[:, nan_cols] = True
    elif base == "blockscale":
        sa[1, nan_rows] = np.nan  # K block 1 of those rows
        sb[[c // 128 for c in nan_cols], 2] = np.nan  # K block 2 of those 128-column blocks
        for c in nan_cols:
            want[:, (c // 128) * 128:min(n, (c // 128) * 128 + 128)] = True
    else:
        sa[5, nan_rows] = 255  # K group 5 of those rows
        sb[7, nan_cols] = 255
        want[:, nan_cols] = True
    got = par.bf16_bits(par.gpu_gemm(dmm_nan, mode, qa, qb, sa, sb))
    ref = oracle.gemm_a8w8(par.MODE_ID[base], qa, qb, sa, sb)
    got_nan, ref_nan = np.isnan(par.bits_to_f64(got)), np.isnan(par.bits_to_f64(ref))
    assert np.array_equal(ref_nan, want), "the oracle's NaN outputs are the poisoned rows and columns"
    assert np.array_equal(got_nan, want), f"{mode}: {np.count_nonzero(got_nan != want)} outputs differ in NaN-ness"
    assert np.array_equal(got[~want], ref[~want]), f"{mode}: {np.count_nonzero(got[~want] != ref[~want])} finite outputs differ"
