"""The oracle's pins have teeth: each mutant below plants one plausible
mistake in a copy of oracle.c (on the CPU), and the pin suite must fail on
every one of them."""
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = {
    "ptpc_drops_b_scale": ("if (mode == ORC_MODE_PTPC) return ((const float*)sb)[n];",
                           "if (mode == ORC_MODE_PTPC) return 1.0f;"),
    "ptpc_drops_a_scale": (": orc_dec_e4m3(j->qa[m * j->K + k]) * scale_a(j->mode, j->sa, j->M, m, k);",
                           ": orc_dec_e4m3(j->qa[m * j->K + k]);"),
    "blockscale_a_ignores_k_block": ("return ((const float*)sa)[(k / 128) * M + m];",
                                     "return ((const float*)sa)[m];"),
    "blockscale_b_transposed_index": ("return ((const float*)sb)[(n / 128) * (K / 128) + k / 128];",
                                      "return ((const float*)sb)[(k / 128) * ((N + 127) / 128) + n / 128];"),
    "mxfp8_wrong_group": ("return orc_dec_e8m0(((const uint8_t*)sa)[(k / 32) * M + m]);",
                          "return orc_dec_e8m0(((const uint8_t*)sa)[(k / 64) * M + m]);"),
    "b_operand_transposed": ("bt[k * N + n] = orc_dec_e4m3(qb[n * K + k])",
                             "bt[k * N + n] = orc_dec_e4m3(qb[k * N + n])"),
    "bf16_truncates": ("return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);",
                       "return (uint16_t)(u >> 16);"),
    "e4m3_ties_away": ("float frac8 = nearbyintf(", "float frac8 = roundf("),
    "e4m3_subnormal_exponent": ("mag = ldexpf((float)f, -9);", "mag = ldexpf((float)f, -8);"),
    "quantiser_multiplies": ("q[r * cols + c] = orc_enc_e4m3(xr[c] / s);",
                             "q[r * cols + c] = orc_enc_e4m3(xr[c] * s);"),
    "mx_exponent_floor": ("e = (fr == 0.5f) ? ex - 1 : ex;", "e = ex - 1;"),
    "accumulate_drops_last_k": ("for (int64_t k = 0; k < j->K; ++k) {\n            const float a",
                                "for (int64_t k = 0; k + 1 < j->K; ++k) {\n            const float a"),
}

PIN_TESTS = [(n, f) for n, f in inspect.getmembers(pins, inspect.isfunction) if n.startswith("test_")]


def _call_all_pins():
    """Run every pin against the currently loaded library; return failures."""
    failed = []
    for name, fn in PIN_TESTS:
        params = getattr(fn, "pytestmark", [])
        cases = [dict()]
        for mark in params:
            if mark.name == "parametrize":
                argnames, argvalues = mark.args[0], mark.args[1]
                names = [a.strip() for a in argnames.split(",")]
                cases = [dict(c, **dict(zip(names, v if len(names) > 1 else (v,)))) for c in cases for v in argvalues]
        for kw in cases:
            try:
                fn(oracle, **kw)
            except AssertionError:
                failed.append((name, kw))
                break
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, tmp_path):
    old, new = MUTANTS[mutant]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {mutant} not found exactly once"
    mpath = tmp_path / "oracle_mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_mutant.so")
    subprocess.run(["gcc", *oracle.CFLAGS, str(mpath), "-o", lib, "-lm"], check=True)
    with oracle.use_library(lib):
        failed = _call_all_pins()
    assert failed, f"no pin caught mutant {mutant}"


def test_unmutated_oracle_passes_the_same_harness():
    assert _call_all_pins() == []
