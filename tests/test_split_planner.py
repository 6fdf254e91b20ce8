"""The split launch's planner (attn_split_grid, host code in the library),
called through its exported symbol on the CPU and checked against the work
partition the kernel uses: workgroup w of a grid of G owns the (query tile,
64-key tile) units [T*w/G, T*(w+1)/G) of the T = tiles * key_tiles units.

Whenever the planner picks a grid, that partition must give every workgroup
work, cover every unit once and cut no query tile into more than four
pieces (the workspace holds four partial slots per tile); the grid must be
whole waves of one workgroup per compute unit.  Whenever it declines, one of
its documented reasons must hold."""

import ctypes
import itertools

import pytest

from attention_attn_block_amd import binding

KEYS_PER_TILE = 64
MAX_PIECES = 4


@pytest.fixture(scope="module")
def planner():
    lib = binding.load()
    fn = getattr(lib, "_ZN3dit15attn_split_gridExiii")
    fn.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    fn.restype = ctypes.c_int
    return fn


def partition(total, grid):
    return [(total * w // grid, total * (w + 1) // grid) for w in range(grid)]


def max_pieces(n_items, n_all, grid):
    total = n_items * n_all
    worst = 0
    for i in range(n_items):
        lo, hi = i * n_all, (i + 1) * n_all
        worst = max(worst, sum(1 for a, b in partition(total, grid) if a < hi and b > lo))
    return worst


def check(planner, n_items, nkv, n_cu, min_tiles):
    grid = planner(n_items, nkv, n_cu, min_tiles)
    n_all = -(-nkv // KEYS_PER_TILE)
    total = n_items * n_all
    if grid == 0:
        waves = -(-n_items // n_cu)
        g = waves * n_cu
        reasons = [n_all < 4, n_all < min_tiles, n_items * 100 >= g * 95, total < g]
        if not any(reasons):
            assert max_pieces(n_items, n_all, g) > MAX_PIECES, (n_items, nkv, n_cu, min_tiles)
        return 0
    assert grid % n_cu == 0 and grid >= n_items
    assert n_items * 100 < grid * 95, "the plain grid already fills its waves"
    assert n_all >= max(4, min_tiles)
    parts = partition(total, grid)
    assert all(b > a for a, b in parts), "every workgroup has work"
    assert parts[0][0] == 0 and parts[-1][1] == total
    assert all(parts[w][1] == parts[w + 1][0] for w in range(grid - 1)), "units covered once"
    assert max_pieces(n_items, n_all, grid) <= MAX_PIECES
    return grid


def test_workloads(planner):
    # 24 heads x 2048 queries against one 2048-key ring block: too short to
    # split unless forced; forced, one wave of 256 workgroups.
    assert check(planner, 192, 2048, 256, 96) == 0
    assert check(planner, 192, 2048, 256, 0) == 256
    # 20 heads x 2048 queries x 16384 keys: split over 256 workgroups.
    assert check(planner, 160, 16384, 256, 96) == 256
    # The video patch (768 tiles: three full waves) keeps the plain grid.
    assert check(planner, 768, 32768, 256, 96) == 0
    # Ulysses share at P = 8 (3 heads x 32768 queries: 384 tiles) and the P = 8
    # PipeFusion patch (24 heads x 4096 queries): two waves of 256.
    assert check(planner, 384, 32768, 256, 96) == 512
    assert check(planner, 384, 32768, 256, 0) == 512


def test_declines(planner):
    assert planner(0, 4096, 256, 0) == 0
    assert planner(10, 4096, 0, 0) == 0
    assert planner(10, 3 * KEYS_PER_TILE, 256, 0) == 0      # fewer than 4 key tiles
    assert planner(10, 50 * KEYS_PER_TILE, 256, 96) == 0    # shorter than the threshold
    assert planner(250, 100 * KEYS_PER_TILE, 256, 0) == 0   # plain grid fills 97.7%


@pytest.mark.parametrize("n_cu", [256, 80, 7])
def test_partition_properties(planner, n_cu):
    items = [1, 2, 3, 5, 31, 100, 191, 192, 255, 257, 300]
    keys = [256, 257, 640, 777, 2048, 4096, 6144, 16384]
    for n_items, nkv, min_tiles in itertools.product(items, keys, (0, 96)):
        check(planner, n_items, nkv, n_cu, min_tiles)
