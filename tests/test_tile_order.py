"""CPU checks of the persistent grid's tile order (``tile_order.h``), compiled
into a host shim with g++: every order visits every output tile exactly once,
and the gathered order (mori PR 809, How it works: tile order) computes the
resident slab first, then each chunk of the other sources in rotation, so a
workgroup's waits only ever move forward."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_matmul_amd", "csrc")

SHIM = r"""
#include "tile_order.h"
using namespace dmm;
extern "C" {
void xcd_list(int wg, int grid, int T, int* o) { auto L = order::xcd_list(wg, grid, T); o[0] = L.first; o[1] = L.stride; o[2] = L.n; }
void round_list(int wg, int grid, int T, int* o) { auto L = order::round_list(wg, grid, T); o[0] = L.first; o[1] = L.stride; o[2] = L.n; }
void coords(int t, int rows_t, int tiles_n, int* o) { order::coords(t, rows_t, tiles_n, o[0], o[1]); }
void gathered(int u, int bt, int nsrc, int nchunks, int own, int tiles_n, int* o) {
    order::gathered_coords(u, bt, nsrc, nchunks, own, tiles_n, o[0], o[1], o[2]);
}
}
"""


@pytest.fixture(scope="module")
def L(tmp_path_factory):
    d = tmp_path_factory.mktemp("order")
    src = d / "shim.cpp"
    src.write_text(SHIM)
    lib = d / "libshim.so"
    subprocess.run(["g++", "-std=c++20", "-O1", "-shared", "-fPIC", "-I", CSRC, str(src), "-o", str(lib)], check=True)
    return ctypes.CDLL(str(lib))


def call(fn, *args, n=3):
    out = (ctypes.c_int * n)()
    fn(*args, out)
    return list(out)


def positions(L, fn, grid, T):
    """Per workgroup, the positions it computes, in order."""
    res = []
    for wg in range(grid):
        first, stride, n = call(fn, wg, grid, T)
        res.append([first + j * stride for j in range(n)])
    return res


@pytest.mark.parametrize("grid,T", [(256, 3584), (256, 448), (256, 3200), (100, 1000), (8, 8), (256, 40),
                                    (13, 97), (256, 257), (224, 224), (896, 896), (1000, 1000)])
@pytest.mark.parametrize("kind", ["xcd_list", "round_list"])
def test_every_position_once(L, kind, grid, T):
    grid = min(grid, T)  # the launch never starts more workgroups than tiles
    got = sorted(p for ps in positions(L, getattr(L, kind), grid, T) for p in ps)
    assert got == list(range(T))


@pytest.mark.parametrize("grid,T", [(256, 3584), (256, 3200), (100, 1000), (13, 97)])
def test_round_list_walks_the_order_front_to_back(L, grid, T):
    """Tile j of every workgroup lies in round j, so the whole grid finishes
    one round of positions before it needs the next."""
    for ps in positions(L, L.round_list, grid, T):
        for j, p in enumerate(ps):
            assert j * grid <= p < (j + 1) * grid


@pytest.mark.parametrize("grid,T", [(256, 3584), (256, 1920)])
def test_xcd_list_keeps_an_xcd_on_neighbouring_positions(L, grid, T):
    for wg, ps in enumerate(positions(L, L.xcd_list, grid, T)):
        x = wg % 8
        lo, hi = x * T // 8 - 1, (x + 1) * T // 8 + 1
        assert all(lo <= p <= hi for p in ps)


@pytest.mark.parametrize("rows_t,tiles_n", [(128, 28), (16, 25), (5, 3), (1, 1), (7, 4)])
def test_coords_is_a_bijection(L, rows_t, tiles_n):
    seen = {tuple(call(L.coords, t, rows_t, tiles_n, n=2)) for t in range(rows_t * tiles_n)}
    assert seen == {(r, c) for r in range(rows_t) for c in range(tiles_n)}


@pytest.mark.parametrize("bt,nsrc,nchunks,own,tiles_n", [(16, 8, 4, 3, 25), (16, 8, 1, 0, 15), (4, 4, 2, 1, 5),
                                                          (2, 2, 2, 1, 3), (8, 1, 1, 0, 7), (16, 8, 16, 7, 2)])
def test_gathered_order(L, bt, nsrc, nchunks, own, tiles_n):
    T = bt * nsrc * tiles_n
    ct = bt // nchunks
    seq = [call(L.gathered, u, bt, nsrc, nchunks, own, tiles_n) for u in range(T)]
    # a bijection onto the tiles
    assert {(tm, tn) for tm, tn, _ in seq} == {(r, c) for r in range(bt * nsrc) for c in range(tiles_n)}
    # the resident slab first, never waiting
    own_part = seq[: bt * tiles_n]
    assert all(band == -1 and own * bt <= tm < (own + 1) * bt for tm, _, band in own_part)
    assert all(band >= 0 for _, _, band in seq[bt * tiles_n:])
    # every other tile waits for the band that holds its rows
    for tm, _, band in seq[bt * tiles_n:]:
        src, c = divmod(band, nchunks)
        assert src != own
        assert src * bt + c * ct <= tm < src * bt + (c + 1) * ct
    # bands come chunk by chunk, sources rotated from own + 1, each band's
    # tiles contiguous
    bands = [b for _, _, b in seq[bt * tiles_n:]]
    order = [b for i, b in enumerate(bands) if i == 0 or b != bands[i - 1]]
    want = [((own + r) % nsrc) * nchunks + c for c in range(nchunks) for r in range(1, nsrc)]
    assert order == want
