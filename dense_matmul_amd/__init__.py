"""Python binding of libdmm (MI355X / gfx950 fp8 a8w8 GEMM).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI of ``include/dmm.h``.  torch supplies device memory and the
current stream; there is no CPU fallback, and every call raises if the
library is not built or the device is not a gfx950.

Functions (names as in the C ABI):
    quantize_per_token(x)             -> (q e4m3 [R,C], scale fp32 [R]); x fp32 or bf16
    quantize_blockscale_a(x)          -> (q, scale fp32 [K/128, M])
    quantize_blockscale_b(x)          -> (q, scale fp32 [ceil(N/128), K/128])
    quantize_mxfp8(x)                 -> (q, scale e8m0 uint8 [K/32, R])
    preshuffle_b(b)                   -> b_shuf (same shape, opaque order)
    gemm_a8w8_ptpc(a, b_shuf, a_scale, b_scale, out=None, tile="auto") -> bf16 [M,N]
        (tile "256x256" / "128x256" calls gemm_a8w8_ptpc_tile)
    gemm_a8w8_ptpc_gathered(a, b_shuf, a_scale, b_scale, flags, src_rows, nchunks, own, epoch,
                            spin_limit=1 << 22, status=None, out=None) -> (bf16 [M,N], status)
    gemm_a8w8_blockscale(a, b_shuf, a_scale, b_scale, out=None) -> bf16 [M,N]
    gemm_a8w8_mxfp8(a, b_shuf, a_scale, b_scale, out=None, tile="auto") -> bf16 [M,N]
        (tile "256x256" / "256x128" calls gemm_a8w8_mxfp8_tile)
    gemm_bf16(a, b, out=None, tile="auto")                       -> bf16 [M,N]

Argument errors (status DMM_EINVAL) raise ValueError; everything else raises
RuntimeError.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdmm.so")

DMM_OK, DMM_EINVAL, DMM_ENODEV, DMM_ELAUNCH = 0, 1, 2, 3

EXPORTS = (
    "dmm_status_str", "dmm_last_error", "quantize_per_token", "quantize_per_token_bf16", "quantize_blockscale_a",
    "quantize_blockscale_b", "quantize_mxfp8", "preshuffle_b", "gemm_a8w8_ptpc", "gemm_a8w8_ptpc_tile",
    "gemm_a8w8_ptpc_gathered", "gemm_a8w8_blockscale", "gemm_a8w8_blockscale_tile", "gemm_a8w8_mxfp8",
    "gemm_a8w8_mxfp8_tile", "gemm_bf16", "gemm_bf16_tile",
)

_lib = None


def lib():
    """The loaded libdmm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libdmm.so is not built ({LIB_PATH}); run __graft_entry__.build() or "
                              "python -m dense_matmul_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.dmm_status_str.argtypes = [ctypes.c_int]
        L.dmm_status_str.restype = ctypes.c_char_p
        L.dmm_last_error.argtypes = []
        L.dmm_last_error.restype = ctypes.c_char_p
        for name in ("quantize_per_token", "quantize_per_token_bf16", "quantize_blockscale_a", "quantize_blockscale_b",
                     "quantize_mxfp8"):
            getattr(L, name).argtypes = [P, P, P, I64, I64, P]
        L.preshuffle_b.argtypes = [P, P, I64, I64, P]
        for name in ("gemm_a8w8_ptpc", "gemm_a8w8_blockscale", "gemm_a8w8_mxfp8"):
            getattr(L, name).argtypes = [P, P, P, P, P, I64, I64, I64, P]
        L.gemm_a8w8_ptpc_tile.argtypes = [P, P, P, P, P, I64, I64, I64, ctypes.c_int, P]
        L.gemm_a8w8_mxfp8_tile.argtypes = [P, P, P, P, P, I64, I64, I64, ctypes.c_int, P]
        L.gemm_a8w8_blockscale_tile.argtypes = [P, P, P, P, P, I64, I64, I64, ctypes.c_int, P]
        L.gemm_a8w8_ptpc_gathered.argtypes = [P, P, P, P, P, I64, I64, I64, P, I64, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_uint32, I64, P, P]
        L.gemm_bf16.argtypes = [P, P, P, I64, I64, I64, P]
        L.gemm_bf16_tile.argtypes = [P, P, P, I64, I64, I64, ctypes.c_int, P]
        for name in EXPORTS[2:]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status == DMM_OK:
        return
    L = lib()
    msg = f"{L.dmm_status_str(status).decode()}: {L.dmm_last_error().decode()}"
    if status == DMM_EINVAL:
        raise ValueError(msg)
    raise RuntimeError(msg)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


_FP8 = (torch.float8_e4m3fn, torch.uint8)


def _codes(t, name):
    """e4m3 codes as a uint8 view (accepts float8_e4m3fn or uint8)."""
    if t.dtype not in _FP8:
        raise ValueError(f"{name}: expected float8_e4m3fn or uint8 codes, got {t.dtype}")
    return t.view(torch.uint8)


def _require(t, name, dtype=None, dims=None, cuda=True):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name}: expected {dims} dimensions, got {t.dim()}")
    if cuda and not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


# ------------------------------------------------------------ quantisers
def quantize_per_token(x, q=None, scale=None):
    """Per-row E4M3 quantisation (scale = amax/448) of fp32 or bf16 x [R, C]
    (bf16 calls quantize_per_token_bf16)."""
    _require(x, "x", None, 2)
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"x: expected float32 or bfloat16, got {x.dtype}")
    r, c = x.shape
    q = torch.empty((r, c), dtype=torch.float8_e4m3fn, device=x.device) if q is None else q
    scale = torch.empty(r, dtype=torch.float32, device=x.device) if scale is None else scale
    _require(q, "q", None, 2)
    _require(scale, "scale", torch.float32, 1)
    _shape(q, (r, c), "q")
    _shape(scale, (r,), "scale")
    fn = lib().quantize_per_token if x.dtype == torch.float32 else lib().quantize_per_token_bf16
    _check(fn(_ptr(x), _ptr(_codes(q, "q")), _ptr(scale), r, c, _stream()))
    return q, scale


def quantize_blockscale_a(x):
    """1x128 blockscale quantisation of fp32 A [M, K]: scale [K/128, M]."""
    _require(x, "x", torch.float32, 2)
    m, k = x.shape
    q = torch.empty((m, k), dtype=torch.float8_e4m3fn, device=x.device)
    scale = torch.empty((max(k // 128, 1), m), dtype=torch.float32, device=x.device)
    _check(lib().quantize_blockscale_a(_ptr(x), _ptr(q.view(torch.uint8)), _ptr(scale), m, k, _stream()))
    return q, scale


def quantize_blockscale_b(x):
    """128x128 blockscale quantisation of fp32 B [N, K]: scale [ceil(N/128), K/128]."""
    _require(x, "x", torch.float32, 2)
    n, k = x.shape
    q = torch.empty((n, k), dtype=torch.float8_e4m3fn, device=x.device)
    scale = torch.empty(((n + 127) // 128, max(k // 128, 1)), dtype=torch.float32, device=x.device)
    _check(lib().quantize_blockscale_b(_ptr(x), _ptr(q.view(torch.uint8)), _ptr(scale), n, k, _stream()))
    return q, scale


def quantize_mxfp8(x):
    """mxfp8 quantisation of fp32 x [R, K]: E8M0 scale bytes [K/32, R]."""
    _require(x, "x", torch.float32, 2)
    r, k = x.shape
    q = torch.empty((r, k), dtype=torch.float8_e4m3fn, device=x.device)
    scale = torch.empty((max(k // 32, 1), r), dtype=torch.uint8, device=x.device)
    _check(lib().quantize_mxfp8(_ptr(x), _ptr(q.view(torch.uint8)), _ptr(scale), r, k, _stream()))
    return q, scale


def preshuffle_b(b, out=None):
    """Reorder B [N, K] e4m3 codes into the GEMM's operand order."""
    _require(b, "b", None, 2)
    bu = _codes(b, "b")
    n, k = b.shape
    out = torch.empty((n, k), dtype=b.dtype, device=b.device) if out is None else out
    _require(out, "out", None, 2)
    _shape(out, (n, k), "out")
    _check(lib().preshuffle_b(_ptr(bu), _ptr(_codes(out, "out")), n, k, _stream()))
    return out


# ------------------------------------------------------------------ GEMM
def _gemm_args(a, b_shuf, out):
    _require(a, "a", None, 2)
    _require(b_shuf, "b_shuf", None, 2)
    m, k = a.shape
    n, k2 = b_shuf.shape
    if k != k2:
        raise ValueError(f"a has K={k} but b_shuf has K={k2}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _require(out, "out", torch.bfloat16, 2)
    _shape(out, (m, n), "out")
    return _codes(a, "a"), _codes(b_shuf, "b_shuf"), out, m, n, k


PTPC_TILES = {"256x256": 1, "128x256": 2, "128x128": 3}


def gemm_a8w8_ptpc(a, b_shuf, a_scale, b_scale, out=None, tile="auto"):
    """C = bf16(a_scale[m] * b_scale[n] * sum_k A[m,k] B[n,k]).  tile: "auto"
    (the library's choice), "256x256", "128x256" or "128x128" (same result)."""
    au, bu, out, m, n, k = _gemm_args(a, b_shuf, out)
    _require(a_scale, "a_scale", torch.float32, 1)
    _require(b_scale, "b_scale", torch.float32, 1)
    _shape(a_scale, (m,), "a_scale")
    _shape(b_scale, (n,), "b_scale")
    if tile == "auto":
        _check(lib().gemm_a8w8_ptpc(_ptr(au), _ptr(bu), _ptr(a_scale), _ptr(b_scale), _ptr(out), m, n, k,
                                    _stream()))
    else:
        if tile not in PTPC_TILES:
            raise ValueError(f"tile must be 'auto' or one of {sorted(PTPC_TILES)} (got {tile!r})")
        _check(lib().gemm_a8w8_ptpc_tile(_ptr(au), _ptr(bu), _ptr(a_scale), _ptr(b_scale), _ptr(out), m, n, k,
                                         PTPC_TILES[tile], _stream()))
    return out


def gemm_a8w8_ptpc_gathered(a, b_shuf, a_scale, b_scale, flags, src_rows, nchunks, own, epoch,
                            spin_limit=1 << 22, status=None, out=None):
    """ptpc GEMM over a gathered A whose source slabs arrive in bands (see
    include/dmm.h).  flags: int32 [m // src_rows * nchunks], on the GPU or in
    pinned host memory (a host thread may write it while the kernel runs);
    band s * nchunks + c is read once (int32)(flags[band] - epoch) >= 0.
    Returns (out, status): status is a GPU int32 [1], 0 unless a band's wait
    gave up after spin_limit polls (then 1 + that band, the largest)."""
    au, bu, out, m, n, k = _gemm_args(a, b_shuf, out)
    _require(a_scale, "a_scale", torch.float32, 1)
    _require(b_scale, "b_scale", torch.float32, 1)
    _shape(a_scale, (m,), "a_scale")
    _shape(b_scale, (n,), "b_scale")
    _require(flags, "flags", torch.int32, 1, cuda=False)
    if not flags.is_cuda and not flags.is_pinned():
        raise ValueError("flags: expected a GPU tensor or pinned host memory")
    if src_rows < 1 or m % src_rows:
        raise ValueError(f"m={m} is not a multiple of src_rows={src_rows}")
    _shape(flags, (m // src_rows * nchunks,), "flags")
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=a.device)
    _require(status, "status", torch.int32, 1)
    _check(lib().gemm_a8w8_ptpc_gathered(_ptr(au), _ptr(bu), _ptr(a_scale), _ptr(b_scale), _ptr(out), m, n, k,
                                         _ptr(flags), src_rows, nchunks, own, epoch & 0xFFFFFFFF, spin_limit,
                                         _ptr(status), _stream()))
    return out, status


BLOCKSCALE_TILES = {"128x256": 1, "128x128": 2}


def gemm_a8w8_blockscale(a, b_shuf, a_scale, b_scale, out=None, tile="auto"):
    """Blockscale GEMM: a_scale [K/128, M] fp32, b_scale [ceil(N/128), K/128] fp32.
    tile: "auto" (the library's choice), "128x256" or "128x128" (same result)."""
    au, bu, out, m, n, k = _gemm_args(a, b_shuf, out)
    _require(a_scale, "a_scale", torch.float32, 2)
    _require(b_scale, "b_scale", torch.float32, 2)
    _shape(a_scale, (k // 128, m), "a_scale")
    _shape(b_scale, ((n + 127) // 128, k // 128), "b_scale")
    args = (_ptr(au), _ptr(bu), _ptr(a_scale), _ptr(b_scale), _ptr(out), m, n, k)
    if tile == "auto":
        _check(lib().gemm_a8w8_blockscale(*args, _stream()))
    else:
        if tile not in BLOCKSCALE_TILES:
            raise ValueError(f"tile must be 'auto' or one of {sorted(BLOCKSCALE_TILES)} (got {tile!r})")
        _check(lib().gemm_a8w8_blockscale_tile(*args, BLOCKSCALE_TILES[tile], _stream()))
    return out


MXFP8_TILES = {"256x256": 1, "256x128": 2}


def gemm_a8w8_mxfp8(a, b_shuf, a_scale, b_scale, out=None, tile="auto"):
    """mxfp8 GEMM: E8M0 scale bytes a_scale [K/32, M], b_scale [K/32, N].
    tile: "auto" (the library's choice), "256x256" or "256x128" (same result)."""
    au, bu, out, m, n, k = _gemm_args(a, b_shuf, out)
    for t, name, rows in ((a_scale, "a_scale", m), (b_scale, "b_scale", n)):
        _require(t, name, None, 2)
        if t.dtype not in (torch.uint8, torch.float8_e8m0fnu):
            raise ValueError(f"{name}: expected uint8 or float8_e8m0fnu, got {t.dtype}")
        _shape(t, (k // 32, rows), name)
    sa, sb = _ptr(a_scale.view(torch.uint8)), _ptr(b_scale.view(torch.uint8))
    if tile == "auto":
        _check(lib().gemm_a8w8_mxfp8(_ptr(au), _ptr(bu), sa, sb, _ptr(out), m, n, k, _stream()))
    else:
        if tile not in MXFP8_TILES:
            raise ValueError(f"tile must be 'auto' or one of {sorted(MXFP8_TILES)} (got {tile!r})")
        _check(lib().gemm_a8w8_mxfp8_tile(_ptr(au), _ptr(bu), sa, sb, _ptr(out), m, n, k, MXFP8_TILES[tile],
                                          _stream()))
    return out


BF16_TILES = {"128x128": 1, "64x64": 2}


def gemm_bf16(a, b, out=None, tile="auto"):
    """C = bf16(sum_k a[m,k] b[n,k]) with fp32 accumulation; a [M,K], b [N,K] bf16.
    tile: "auto", "128x128" or "64x64" (same result)."""
    _require(a, "a", torch.bfloat16, 2)
    _require(b, "b", torch.bfloat16, 2)
    m, k = a.shape
    n, k2 = b.shape
    if k != k2:
        raise ValueError(f"a has K={k} but b has K={k2}")
    out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device) if out is None else out
    _require(out, "out", torch.bfloat16, 2)
    _shape(out, (m, n), "out")
    if tile == "auto":
        _check(lib().gemm_bf16(_ptr(a), _ptr(b), _ptr(out), m, n, k, _stream()))
    else:
        if tile not in BF16_TILES:
            raise ValueError(f"tile must be 'auto' or one of {sorted(BF16_TILES)} (got {tile!r})")
        _check(lib().gemm_bf16_tile(_ptr(a), _ptr(b), _ptr(out), m, n, k, BF16_TILES[tile], _stream()))
    return out
