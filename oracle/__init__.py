"""CPU oracle for the fp8 a8w8 GEMM -- TEST INFRASTRUCTURE ONLY.

Thin ctypes/numpy wrapper over ``oracle.c`` (plain C, built with gcc, no
contraction, no fast-math).  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package; the product
library never does, and the two share no code.

What is computed, and where the pages define it, is stated in ``oracle.c``:
dequantise each operand to fp32, accumulate in fp32 in ascending k, round
the result to bf16 (mori PR 785, section Test; aiter PR 6539, Test Plan).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

MODE_PTPC, MODE_BLOCKSCALE, MODE_MXFP8 = 0, 1, 2
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared", "-pthread"]


def build(lib: str = LIB, extra: tuple = ()) -> str:
    """Compile oracle.c with gcc into ``lib`` (always recompiles)."""
    tmp = lib + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _bind(L):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    for name in ("orc_dec_e4m3_n", "orc_enc_e4m3_n", "orc_dec_e8m0_n", "orc_bf16_rne_n", "orc_bf16_to_f32_n"):
        getattr(L, name).argtypes = [P, P, I64]
        getattr(L, name).restype = None
    L.orc_quantize_rows.argtypes = [P, I64, I64, P, P]
    L.orc_quantize_blockscale_a.argtypes = [P, I64, I64, P, P]
    L.orc_quantize_blockscale_b.argtypes = [P, I64, I64, P, P]
    L.orc_quantize_mxfp8.argtypes = [P, I64, I64, P, P]
    for name in ("orc_quantize_rows", "orc_quantize_blockscale_a", "orc_quantize_blockscale_b", "orc_quantize_mxfp8"):
        getattr(L, name).restype = None
    L.orc_gemm_a8w8.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, I64, P, I64, P, P, ctypes.c_int]
    L.orc_gemm_a8w8.restype = ctypes.c_int
    L.orc_gemm_bf16.argtypes = [P, P, I64, I64, I64, P, I64, P, P, ctypes.c_int]
    L.orc_gemm_bf16.restype = ctypes.c_int
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _elementwise(fn, x, in_dtype, out_dtype):
    x = _c(x, in_dtype)
    out = np.empty(x.shape, dtype=out_dtype)
    getattr(_load(), fn)(_ptr(x), _ptr(out), x.size)
    return out


# ------------------------------------------------------------------ codecs
def dec_e4m3(q):
    """OCP FP8 E4M3 code -> float32 value (NaN for S.1111.111)."""
    return _elementwise("orc_dec_e4m3_n", q, np.uint8, np.float32)


def enc_e4m3(x):
    """float32 -> E4M3 code, round to nearest even, saturate to +-448."""
    return _elementwise("orc_enc_e4m3_n", x, np.float32, np.uint8)


def dec_e8m0(b):
    """OCP MX E8M0 scale byte -> 2^(b-127) (NaN for 255)."""
    return _elementwise("orc_dec_e8m0_n", b, np.uint8, np.float32)


def bf16_rne(x):
    """float32 -> bf16 bit pattern (uint16), round to nearest even."""
    return _elementwise("orc_bf16_rne_n", x, np.float32, np.uint16)


def bf16_to_f32(h):
    return _elementwise("orc_bf16_to_f32_n", h, np.uint16, np.float32)


# -------------------------------------------------------------- quantisers
def quantize_rows(x):
    """Per-row e4m3 quantisation with scale amax/448: per token for A [M,K],
    per output channel for B [N,K].  Returns (codes uint8, scale float32[rows])."""
    x = _c(x, np.float32)
    r, c = x.shape
    q = np.empty((r, c), np.uint8)
    s = np.empty(r, np.float32)
    _load().orc_quantize_rows(_ptr(x), r, c, _ptr(q), _ptr(s))
    return q, s


quantize_per_token = quantize_rows


def quantize_blockscale_a(x):
    """1x128 blocks: returns (codes [M,K], scale float32 [K/128, M])."""
    x = _c(x, np.float32)
    m, k = x.shape
    assert k % 128 == 0
    q = np.empty((m, k), np.uint8)
    s = np.empty((k // 128, m), np.float32)
    _load().orc_quantize_blockscale_a(_ptr(x), m, k, _ptr(q), _ptr(s))
    return q, s


def quantize_blockscale_b(x):
    """128x128 blocks: returns (codes [N,K], scale float32 [ceil(N/128), K/128])."""
    x = _c(x, np.float32)
    n, k = x.shape
    assert k % 128 == 0
    q = np.empty((n, k), np.uint8)
    s = np.empty(((n + 127) // 128, k // 128), np.float32)
    _load().orc_quantize_blockscale_b(_ptr(x), n, k, _ptr(q), _ptr(s))
    return q, s


def quantize_mxfp8(x):
    """E8M0 scale per 32 K values: returns (codes [R,K], scale bytes uint8 [K/32, R])."""
    x = _c(x, np.float32)
    r, k = x.shape
    assert k % 32 == 0
    q = np.empty((r, k), np.uint8)
    e = np.empty((k // 32, r), np.uint8)
    _load().orc_quantize_mxfp8(_ptr(x), r, k, _ptr(q), _ptr(e))
    return q, e


# -------------------------------------------------------------------- GEMM
def gemm_a8w8(mode, qa, qb, sa, sb, rows=None, threads=0, want_f32=False):
    """C[rows, :] of the fp8 a8w8 GEMM in ``mode``.  qa [M,K] and qb [N,K] are
    E4M3 codes (B not preshuffled).  Returns bf16 bits uint16 [len(rows), N],
    plus the unrounded fp32 sums when ``want_f32``."""
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    M, K = qa.shape
    N, K2 = qb.shape
    assert K == K2
    sdt = np.uint8 if mode == MODE_MXFP8 else np.float32
    sa = _c(sa, sdt)
    sb = _c(sb, sdt)
    if rows is not None:
        rows = _c(rows, np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < M)
    nr = M if rows is None else rows.size
    c = np.empty((nr, N), np.uint16)
    c32 = np.empty((nr, N), np.float32) if want_f32 else None
    used = _load().orc_gemm_a8w8(mode, _ptr(qa), _ptr(qb), _ptr(sa), _ptr(sb), M, N, K, _ptr(rows),
                                 nr, _ptr(c), _ptr(c32), threads)
    if used < 0:
        raise MemoryError("oracle GEMM failed to allocate")
    return (c, c32) if want_f32 else c


def gemm_ptpc(qa, qb, a_scale, b_scale, **kw):
    return gemm_a8w8(MODE_PTPC, qa, qb, a_scale, b_scale, **kw)


def gemm_blockscale(qa, qb, a_scale, b_scale, **kw):
    return gemm_a8w8(MODE_BLOCKSCALE, qa, qb, a_scale, b_scale, **kw)


def gemm_mxfp8(qa, qb, a_scale, b_scale, **kw):
    return gemm_a8w8(MODE_MXFP8, qa, qb, a_scale, b_scale, **kw)


def gemm_bf16(a, b, rows=None, threads=0, want_f32=False):
    """bf16 [M,K] x bf16 [N,K]^T (bit patterns as uint16), fp32 accumulate."""
    a = _c(a, np.uint16)
    b = _c(b, np.uint16)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    if rows is not None:
        rows = _c(rows, np.int64)
    nr = M if rows is None else rows.size
    c = np.empty((nr, N), np.uint16)
    c32 = np.empty((nr, N), np.float32) if want_f32 else None
    used = _load().orc_gemm_bf16(_ptr(a), _ptr(b), M, N, K, _ptr(rows), nr, _ptr(c), _ptr(c32), threads)
    if used < 0:
        raise MemoryError("oracle GEMM failed to allocate")
    return (c, c32) if want_f32 else c


def threads_available():
    return os.cpu_count() or 1


class use_library:
    """Context manager that routes this module's calls to another build of
    oracle.c (the mutation tests build deliberately broken copies)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False
