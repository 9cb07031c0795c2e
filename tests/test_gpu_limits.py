"""The GEMMs at the operand-size limits of the C ABI.

Operands are addressed with 32-bit buffer offsets, so the C ABI takes A, B
and C up to 2^31 bytes each, with a margin of 256 rows (the rows a last tile
may reach past M or N).  Each test drives one operand to that limit:

* A: M = 299337, N = 16, K = 7168 (A 2.146 GB), every tile of every mode;
* B: M = 1, N = 4177968, K = 512 (B 2.139 GB, and its preshuffled copy),
  ptpc on its three tiles and mxfp8 on its two;
* C: M = 149540, N = 7168, K = 128 (C 2.144 GB), every tile of every mode;
* and the bf16 GEMM's three limits (A 1048319 x 1024, B 1048304 x 1024, C
  149540 x 7168), both tiles.

The data sit in the exact regime (values 0, +-0.5, +-1, +-2 and power-of-two
scales), where every sum is exact in fp32, so the GPU must equal the oracle
bit for bit.  The large operand is drawn on the device by torch's seeded
generator; the oracle gets the sampled rows (or 128-column blocks) copied
back, with the small operand and the scales from the host generators.  C is
NaN-poisoned and followed by a canary before each launch: every element must
be written and nothing past C.
"""
import numpy as np
import pytest
import torch

import oracle
from dense_matmul_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LIMIT = 1 << 31
MODE_ID = {"ptpc": 0, "blockscale": 1, "mxfp8": 2}
P2 = np.array([0.25, 0.5, 1.0, 2.0, 4.0], np.float32)
E8M0 = np.arange(125, 130, dtype=np.uint8)
TILES = {"ptpc": ("256x256", "128x256", "128x128"), "mxfp8": ("256x256", "256x128"), "blockscale": ("128x256", "128x128")}

# OCP E4M3 codes of 0.5, 1 and 2 (exponent bias 7), sign in bit 7
MAG_CODES = (0x30, 0x38, 0x40)


@pytest.fixture(scope="module")
def dmm():
    import dense_matmul_amd as d

    d.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return d


def test_magnitude_codes_decode_to_the_exact_values():
    vals = oracle.dec_e4m3(np.array(MAG_CODES + tuple(c | 0x80 for c in MAG_CODES) + (0,), np.uint8))
    assert vals.tolist() == [0.5, 1.0, 2.0, -0.5, -1.0, -2.0, 0.0]


def exact_codes_device(shape, seed):
    """uint8 codes on the device, each 0 (with either sign) or +-0.5, +-1, +-2,
    drawn by torch's generator seeded with ``seed``."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    r = torch.randint(0, 4, shape, generator=g, device=DEV, dtype=torch.uint8)
    s = torch.randint(0, 2, shape, generator=g, device=DEV, dtype=torch.uint8)
    # r = 1, 2, 3 -> 0x30, 0x38, 0x40; r = 0 -> 0
    code = torch.where(r > 0, r * 8 + 0x28, torch.zeros_like(r))
    del r
    return code | (s << 7)


def exact_codes_host(shape, seed):
    vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0], np.float32)
    return inputs.choice(shape, oracle.enc_e4m3(vals), seed)


def scales(mode, m, n, k, seed):
    if mode == "ptpc":
        return inputs.choice((m,), P2, seed), inputs.choice((n,), P2, seed + 1)
    if mode == "blockscale":
        return inputs.choice((k // 128, m), P2, seed), inputs.choice(((n + 127) // 128, k // 128), P2, seed + 1)
    return inputs.choice((k // 32, m), E8M0, seed), inputs.choice((k // 32, n), E8M0, seed + 1)


def gemm(dmm, mode):
    return {"ptpc": dmm.gemm_a8w8_ptpc, "mxfp8": dmm.gemm_a8w8_mxfp8, "blockscale": dmm.gemm_a8w8_blockscale}[mode]


def run_poisoned(dmm, mode, tile, a, b_shuf, sa, sb, m, n):
    buf = torch.empty(m * n + 2048, dtype=torch.bfloat16, device=DEV)
    c = buf[: m * n].view(m, n)
    canary = buf[m * n:].view(torch.int16)
    buf.fill_(float("nan"))
    canary.fill_(0x5A5A)
    gemm(dmm, mode)(a, b_shuf, sa, sb, out=c, tile=tile)
    torch.cuda.synchronize()
    assert not torch.isnan(c).any().item(), f"{mode} {tile}: unwritten elements"
    assert bool((canary == 0x5A5A).all().item()), f"{mode} {tile}: write past the end of C"
    return c


def assert_bitwise(got, ref, what):
    bad = np.count_nonzero(got != ref)
    assert bad == 0, f"{what}: {bad} of {ref.size} sampled elements differ from the oracle"
    print(f"[bitwise] {what}: {ref.size} sampled elements equal the oracle", flush=True)


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("mode", ["ptpc", "mxfp8", "blockscale"])
def test_a_at_the_limit(dmm, mode):
    m, n, k = 299337, 16, 7168
    assert (m + 256) * k < LIMIT <= (m + 257) * k
    print(f"[case] limits A {mode} {m}x{n}x{k}", flush=True)
    a = exact_codes_device((m, k), 701)
    qb = exact_codes_host((n, k), 702)
    sa, sb = scales(mode, m, n, k, 703)
    b_shuf = dmm.preshuffle_b(torch.from_numpy(qb).to(DEV))
    s_a, s_b = torch.from_numpy(np.ascontiguousarray(sa)).to(DEV), torch.from_numpy(sb).to(DEV)
    rows = inputs.rows_sample(m, seed=704)
    qa_rows = a[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    sa_rows = sa[rows] if mode == "ptpc" else np.ascontiguousarray(sa[:, rows])
    ref = oracle.gemm_a8w8(MODE_ID[mode], qa_rows, qb, sa_rows, sb)
    for tile in TILES[mode]:
        c = run_poisoned(dmm, mode, tile, a, b_shuf, s_a, s_b, m, n)
        assert_bitwise(bits(c[torch.from_numpy(rows).to(DEV)]), ref, f"A limit {mode} {tile}")
        del c
    del a, b_shuf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["ptpc", "mxfp8"])
def test_b_at_the_limit(dmm, mode):
    m, n, k = 1, 4177968, 512
    assert n % 16 == 0 and (n + 256) * k < LIMIT and (m + 256) * n * 2 < LIMIT
    print(f"[case] limits B {mode} {m}x{n}x{k}", flush=True)
    b = exact_codes_device((n, k), 711)
    qa = exact_codes_host((m, k), 712)
    sa, sb = scales(mode, m, n, k, 713)
    b_shuf = dmm.preshuffle_b(b)
    a, s_a, s_b = (torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in (qa, sa, sb))
    # whole 128-column blocks: the first two, the last two, and 16 drawn ones
    nblk = n // 128
    blocks = sorted({0, 1, nblk - 2, nblk - 1, *np.random.default_rng(714).integers(0, nblk, 16).tolist()})
    cols = np.concatenate([np.arange(128 * j, 128 * j + 128) for j in blocks])
    tail = np.arange(128 * nblk, n)  # the columns past the last whole block
    cols = np.concatenate([cols, tail])
    qb_cols = b[torch.from_numpy(cols).to(DEV)].cpu().numpy()
    sb_cols = sb[cols] if mode == "ptpc" else np.ascontiguousarray(sb[:, cols])
    ref = oracle.gemm_a8w8(MODE_ID[mode], qa, qb_cols, sa, sb_cols)
    del b
    for tile in TILES[mode]:
        c = run_poisoned(dmm, mode, tile, a, b_shuf, s_a, s_b, m, n)
        assert_bitwise(bits(c[:, torch.from_numpy(cols).to(DEV)]), ref, f"B limit {mode} {tile}")
        del c
    del b_shuf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["ptpc", "mxfp8", "blockscale"])
def test_c_at_the_limit(dmm, mode):
    m, n, k = 149540, 7168, 128
    assert (m + 256) * n * 2 < LIMIT <= (m + 257) * n * 2
    print(f"[case] limits C {mode} {m}x{n}x{k}", flush=True)
    qa = exact_codes_host((m, k), 721)
    qb = exact_codes_host((n, k), 722)
    sa, sb = scales(mode, m, n, k, 723)
    a, s_a, s_b = (torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in (qa, sa, sb))
    b_shuf = dmm.preshuffle_b(torch.from_numpy(qb).to(DEV))
    rows = inputs.rows_sample(m, seed=724)
    ref = oracle.gemm_a8w8(MODE_ID[mode], qa, qb, sa, sb, rows=rows)
    for tile in TILES[mode]:
        c = run_poisoned(dmm, mode, tile, a, b_shuf, s_a, s_b, m, n)
        assert_bitwise(bits(c[torch.from_numpy(rows).to(DEV)]), ref, f"C limit {mode} {tile}")
        del c
    torch.cuda.empty_cache()


# bf16 bit patterns of 0.5, 1 and 2 (0x3F00, 0x3F80, 0x4000), sign in bit 15
def test_bf16_patterns_are_the_exact_values():
    h = np.array([0x3F00, 0x3F80, 0x4000, 0xBF00, 0xBF80, 0xC000, 0], np.uint16)
    assert oracle.bf16_to_f32(h).tolist() == [0.5, 1.0, 2.0, -0.5, -1.0, -2.0, 0.0]


def exact_bf16_device(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    r = torch.randint(0, 4, shape, generator=g, device=DEV, dtype=torch.int16)
    s = torch.randint(0, 2, shape, generator=g, device=DEV, dtype=torch.int16)
    h = torch.where(r > 0, r * 0x80 + 0x3E80, torch.zeros_like(r))
    del r
    return (h | (s << 15)).view(torch.bfloat16)


def exact_bf16_host(shape, seed):
    return inputs.choice(shape, np.array([0x3F00, 0x3F80, 0x4000, 0xBF00, 0xBF80, 0xC000, 0], np.uint16), seed)


@pytest.mark.parametrize("which", ["A", "B", "C"])
def test_bf16_at_the_limit(dmm, which):
    m, n, k = {"A": (1048319, 16, 1024), "B": (1, 1048304, 1024), "C": (149540, 7168, 64)}[which]
    assert n % 16 == 0 and k % 64 == 0
    assert (m + 256) * k * 2 < LIMIT and (n + 256) * k * 2 < LIMIT and (m + 256) * n * 2 < LIMIT
    print(f"[case] limits bf16 {which} {m}x{n}x{k}", flush=True)
    dev = lambda h: torch.from_numpy(h.view(np.int16)).to(DEV).view(torch.bfloat16)
    host = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    if which == "A":
        a, qb = exact_bf16_device((m, k), 731), exact_bf16_host((n, k), 732)
        b = dev(qb)
        rows = inputs.rows_sample(m, seed=733)
        ref = oracle.gemm_bf16(host(a[torch.from_numpy(rows).to(DEV)]), qb)
        pick = lambda c: c[torch.from_numpy(rows).to(DEV)]
    elif which == "B":
        qa, b = exact_bf16_host((m, k), 741), exact_bf16_device((n, k), 742)
        a = dev(qa)
        cols = np.unique(np.concatenate([np.arange(256), np.arange(n - 256, n),
                                         np.random.default_rng(743).integers(0, n, 2048)]))
        ref = oracle.gemm_bf16(qa, host(b[torch.from_numpy(cols).to(DEV)]))
        pick = lambda c: c[:, torch.from_numpy(cols).to(DEV)]
    else:
        qa, qb = exact_bf16_host((m, k), 751), exact_bf16_host((n, k), 752)
        a, b = dev(qa), dev(qb)
        rows = inputs.rows_sample(m, seed=753)
        ref = oracle.gemm_bf16(qa, qb, rows=rows)
        pick = lambda c: c[torch.from_numpy(rows).to(DEV)]
    for tile in ("128x128", "64x64"):
        buf = torch.empty(m * n + 2048, dtype=torch.bfloat16, device=DEV)
        c = buf[: m * n].view(m, n)
        canary = buf[m * n:].view(torch.int16)
        buf.fill_(float("nan"))
        canary.fill_(0x5A5A)
        dmm.gemm_bf16(a, b, out=c, tile=tile)
        torch.cuda.synchronize()
        assert not torch.isnan(c).any().item(), f"bf16 {which} {tile}: unwritten elements"
        assert bool((canary == 0x5A5A).all().item()), f"bf16 {which} {tile}: write past the end of C"
        assert_bitwise(host(pick(c).contiguous()), ref, f"bf16 {which} limit {tile}")
        del buf, c, canary
    del a, b
    torch.cuda.empty_cache()


# The quantisers index rows with 64-bit offsets: a per-token, blockscale or
# mxfp8 input of 300000 x 7168 fp32 (2.15e9 values, 8.6 GB, past 2^31 values)
# and a blockscale B of 4177968 x 512 (a partial last 128-row block), N(0,1)
# from torch's seeded generator; sampled rows (whole 128-row blocks for B)
# against the oracle's quantisers, codes and scales bitwise.
@pytest.mark.parametrize("kind", ["per_token", "per_token_bf16", "blockscale_a", "mxfp8", "blockscale_b"])
def test_quantisers_past_2_31_values(dmm, kind):
    m, k = (4177968, 512) if kind == "blockscale_b" else (300000, 7168)
    print(f"[case] limits quantiser {kind} {m}x{k}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(771)
    x = torch.randn((m, k), generator=g, device=DEV, dtype=torch.float32)
    if kind == "per_token_bf16":
        x = x.to(torch.bfloat16)
    fn = {"per_token": dmm.quantize_per_token, "per_token_bf16": dmm.quantize_per_token,
          "blockscale_a": dmm.quantize_blockscale_a, "mxfp8": dmm.quantize_mxfp8,
          "blockscale_b": dmm.quantize_blockscale_b}[kind]
    q, s = fn(x)
    torch.cuda.synchronize()
    if kind == "blockscale_b":
        nblk = (m + 127) // 128
        blocks = sorted({0, nblk - 2, nblk - 1, *np.random.default_rng(772).integers(0, nblk, 8).tolist()})
        rows = np.concatenate([np.arange(128 * j, min(m, 128 * j + 128)) for j in blocks])
    else:
        rows = inputs.rows_sample(m, seed=772)
    rows_t = torch.from_numpy(rows).to(DEV)
    xr = x[rows_t].float().cpu().numpy()
    got_q = q.view(torch.uint8)[rows_t].cpu().numpy()
    if kind.startswith("per_token"):
        ref_q, ref_s = oracle.quantize_per_token(xr)
        got_s = s[rows_t].cpu().numpy()
    elif kind == "blockscale_a":
        ref_q, ref_s = oracle.quantize_blockscale_a(xr)
        got_s = s[:, rows_t].cpu().numpy()
    elif kind == "mxfp8":
        ref_q, ref_s = oracle.quantize_mxfp8(xr)
        got_s = s[:, rows_t].cpu().numpy()
    else:
        ref_q, ref_s = oracle.quantize_blockscale_b(xr)
        got_s = s[torch.tensor(blocks, device=DEV)].cpu().numpy()
    assert_bitwise(got_q, ref_q, f"quantiser {kind} codes")
    assert np.array_equal(got_s.view(np.uint8), np.ascontiguousarray(ref_s).view(np.uint8)), f"{kind}: scales differ"
    del x, q, s
    torch.cuda.empty_cache()
