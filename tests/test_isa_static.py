"""Static checks on the emitted gfx950 code of libdmm (no GPU).

For every kernel of the three device sources, from this build's own code
objects (_build/<src>.o, extracted by dense_matmul_amd.build.disassemble):

* no kernel spills to scratch memory (its code-object metadata states a
  private segment of 0 bytes);
* no kernel uses packed fp32 arithmetic (the build turns the packed-fp32
  target feature off, so the compiler never forms it and nothing is written
  by hand);
* no kernel writes through the scalar data cache: no scalar memory store or
  atomic, no write-back or discard of that cache.  Every store goes through
  the vector memory path.

The mutants at the end edit the texts and must be caught.
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SOURCES = ("gemm_a8w8.hip", "gemm_bf16.hip", "quant.hip")
READELF = "/opt/rocm/llvm/bin/llvm-readelf"
MNEMONIC = re.compile(r"^\s+([a-z_0-9]+)\b.*//\s*[0-9A-F]+:", re.M)
PACKED_FP32 = re.compile(r"^v_pk_(add|mul|fma|mov)_f32")
SCALAR_WRITE = re.compile(r"^s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)")


@pytest.fixture(scope="module")
def code():
    from dense_matmul_amd import build

    out = {}
    for src in SOURCES:
        text = build.disassemble(src)
        co = os.path.join(ROOT, "_build", "disasm", src + ".co")
        notes = subprocess.run([READELF, "--notes", co], capture_output=True, text=True, check=True).stdout
        out[src] = (text, notes)
    return out


def private_segments(notes):
    """{kernel symbol: private segment bytes} from the code object's metadata."""
    names = re.findall(r"^\s+\.name:\s+(_Z\S+)\s*$", notes, re.M)
    sizes = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)]
    assert len(names) == len(sizes), "one private segment size per kernel"
    return dict(zip(names, sizes))


def forbidden(text):
    bad = []
    for mn in MNEMONIC.findall(text):
        if PACKED_FP32.match(mn) or SCALAR_WRITE.match(mn):
            bad.append(mn)
    return bad


def test_no_kernel_spills_to_scratch(code):
    n = 0
    for src, (_, notes) in code.items():
        seg = private_segments(notes)
        assert seg, f"{src}: no kernels in the code object"
        spills = {k: v for k, v in seg.items() if v}
        assert not spills, f"{src}: kernels with scratch: {spills}"
        n += len(seg)
    assert n >= 50, "every GEMM and quantiser kernel was looked at"


def test_no_packed_fp32_and_no_scalar_cache_writes(code):
    for src, (text, _) in code.items():
        insns = MNEMONIC.findall(text)
        assert len(insns) > 1000
        bad = forbidden(text)
        assert not bad, f"{src}: forbidden instructions {sorted(set(bad))}"


def test_checks_catch_planted_instructions(code):
    text, notes = code["quant.hip"]
    line = "\tv_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]                // 000000001234: D3B00000\n"
    assert forbidden(text + line)
    line = "\ts_store_dword s0, s[2:3], 0x0                               // 000000001238: C0420001\n"
    assert forbidden(text + line)
    spilled = notes.replace(".private_segment_fixed_size: 0", ".private_segment_fixed_size: 16", 1)
    assert any(private_segments(spilled).values())
