"""Pins for the oracle's Hilbert index, plans and gather/scatter (CPU only).

The pins come from the mathematics of Hilbert curves and from the plan's
definition, not from the oracle itself: Gray-code base case, unit steps,
octant recursion, endpoints, bijection, and brute-force filtering.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
import workloads as wl


def _cube_order(b):
    S = 1 << b
    cells = np.array(list(itertools.product(range(S), repeat=3)), dtype=np.int64)
    h = oracle.hilbert_index(cells[:, 0], cells[:, 1], cells[:, 2], b)
    return cells, h


def test_order1_is_gray_code(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "hilbert_order1.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                p = line.split()
                rows.append((int(p[0]), tuple(int(c) for c in p[2:5])))
    cells, h = _cube_order(1)
    for i, cell in rows:
        got = tuple(cells[np.nonzero(h == i)[0][0]])
        assert got == cell


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5])
def test_cube_bijection_and_unit_steps(b):
    cells, h = _cube_order(b)
    assert sorted(h.tolist()) == list(range(8 ** b))
    path = cells[np.argsort(h)]
    step = np.abs(np.diff(path, axis=0)).sum(axis=1)
    assert np.all(step == 1), "every step of a Hilbert curve moves to a face neighbour"


@pytest.mark.parametrize("b", [2, 3, 4])
def test_octant_recursion(b):
    """Every aligned run of 8**k consecutive indices fills one aligned cube of
    side 2**k (the self-similarity that separates a Hilbert curve from other
    unit-step orders such as a boustrophedon scan)."""
    cells, h = _cube_order(b)
    path = cells[np.argsort(h)]
    for k in range(1, b):
        run = 8 ** k
        side = 1 << k
        for r in range(0, 8 ** b, run):
            chunk = path[r:r + run]
            lo = chunk.min(axis=0)
            assert np.all(lo % side == 0)
            assert np.all(chunk.max(axis=0) - lo == side - 1)
            assert len({tuple(c) for c in chunk}) == run


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5])
def test_endpoints(b):
    cells, h = _cube_order(b)
    path = cells[np.argsort(h)]
    assert tuple(path[0]) == (0, 0, 0)
    # the curve ends on the corner adjacent to the start along axis 0
    assert tuple(path[-1]) == ((1 << b) - 1, 0, 0)


def test_order_bits():
    assert oracle.hilbert_order_bits(1, 1, 1) == 1
    assert oracle.hilbert_order_bits(8, 16, 16) == 4
    assert oracle.hilbert_order_bits(21, 30, 52) == 6
    assert oracle.hilbert_order_bits(33, 45, 80) == 7


def _brute_filtered_order(T, H, W):
    b = oracle.hilbert_order_bits(T, H, W)
    cells, h = _cube_order(b)
    out = []
    for c in cells[np.argsort(h)]:
        t, y, x = (int(v) for v in c)
        if t < T and y < H and x < W:
            out.append((t * H + y) * W + x)
    return np.array(out)


@pytest.mark.parametrize("shape", [(3, 5, 7), (2, 3, 4), (5, 1, 6), (1, 1, 1), (4, 8, 8)])
def test_hilbert_plan_skips_out_of_grid_cells(shape):
    T, H, W = shape
    B = 4
    perm, blk_len = oracle.plan(T, H, W, "hilbert", B)
    N = T * H * W
    assert np.array_equal(perm[:N], _brute_filtered_order(T, H, W))
    assert np.all(perm[N:] == -1)
    assert perm.size % B == 0 and perm.size - N < B
    assert blk_len.sum() == N


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_plan_is_bijection(idx):
    w = wl.get(idx)
    perm, blk_len = oracle.plan(w.T, w.H, w.W, w.order, w.B)
    real = perm[perm >= 0]
    assert np.array_equal(np.sort(real), np.arange(w.N))
    assert blk_len.sum() == w.N
    assert np.all(blk_len >= 1) and np.all(blk_len <= w.B)
    nb = perm.size // w.B
    assert np.array_equal(blk_len, (perm.reshape(nb, w.B) >= 0).sum(1))


def test_workload_block_counts():
    expect = {1: (4, 64), 2: (32, 64), 3: (256, 120), 4: (793, 24), 5: (929, 16)}
    for idx, (nb, last) in expect.items():
        w = wl.get(idx)
        perm, blk_len = oracle.plan(w.T, w.H, w.W, w.order, w.B)
        assert perm.size // w.B == nb
        assert blk_len[-1] == last


def test_row_and_frame_plans():
    perm, blk = oracle.plan(3, 5, 7, "row", 16)
    assert np.array_equal(perm[:105], np.arange(105)) and np.all(perm[105:] == -1)
    perm, blk = oracle.plan(3, 5, 7, "frame", 16)   # 35 tokens -> 3 tiles per frame
    assert perm.size == 3 * 48
    for f in range(3):
        tile = perm[f * 48:(f + 1) * 48]
        assert np.array_equal(tile[:35], np.arange(f * 35, f * 35 + 35))
        assert np.all(tile[35:] == -1)
    assert blk.tolist() == [16, 16, 3] * 3


def test_cfg2_grid_is_first_half_of_cube_curve():
    """The order-4 curve spends its first half in the half cube t < 8 (its
    first four octants share X0 = 0), so the 8x16x16 grid is a single
    unbroken stretch of the curve with unit steps throughout."""
    w = wl.get(2)
    perm, _ = oracle.plan(w.T, w.H, w.W, "hilbert", w.B)
    t, r = np.divmod(perm, w.H * w.W)
    y, x = np.divmod(r, w.W)
    step = np.abs(np.diff(t)) + np.abs(np.diff(y)) + np.abs(np.diff(x))
    assert np.all(step == 1)


def test_hilbert_blocks_are_more_compact_than_raster():
    """DFSAttn, Methodology, design 1: the reorder keeps spatiotemporal
    neighbourhoods together inside a block; measured as the mean volume of
    each block's bounding box on the Wan 480p latent grid."""
    w = wl.get(3)

    def mean_box(order):
        perm, _ = oracle.plan(w.T, w.H, w.W, order, w.B)
        vols = []
        for I in range(perm.size // w.B):
            p = perm[I * w.B:(I + 1) * w.B]
            p = p[p >= 0]
            t, r = np.divmod(p, w.H * w.W)
            y, x = np.divmod(r, w.W)
            vols.append((np.ptp(t) + 1) * (np.ptp(y) + 1) * (np.ptp(x) + 1))
        return float(np.mean(vols))

    assert mean_box("hilbert") * 2 < mean_box("row")


@pytest.mark.parametrize("idx", [1, 2])
def test_gather_scatter_roundtrip(idx):
    w = wl.get(idx)
    q, _, _ = wl.make_qkv(w, 0)
    perm, _ = oracle.plan(w.T, w.H, w.W, w.order, w.B)
    xp = oracle.gather(q, perm)
    assert np.all(xp[:, perm < 0, :] == 0)
    back = oracle.scatter(xp, perm, w.N)
    assert np.array_equal(back, q.double().numpy())
    inv = oracle.inverse_perm(perm, w.N)
    assert np.array_equal(perm[inv], np.arange(w.N))


# ---------------------------------------------------------------- VMoBA tiled partitions

def _tile_shape(order, B):
    return (1, 8, B // 8) if order == "tile2d" else (B // 64, 8, 8)


def _coords(perm, H, W):
    t, r = np.divmod(perm, H * W)
    y, x = np.divmod(r, W)
    return t, y, x


@pytest.mark.parametrize("order,shape,B", [
    ("tile2d", (3, 5, 7), 64), ("tile2d", (21, 30, 52), 128), ("tile2d", (2, 17, 40), 128),
    ("cube3d", (3, 5, 7), 64), ("cube3d", (21, 30, 52), 128), ("cube3d", (5, 9, 17), 128),
])
def test_tiled_plan_blocks_are_clipped_tiles(order, shape, B):
    """Every real token appears once; block k holds exactly the cells of the
    k-th tile (row-major over tile coordinates, clipped to the grid) in
    row-major order, followed by pads; blk_len is the clipped volume."""
    T, H, W = shape
    N = T * H * W
    perm, blk_len = oracle.plan(T, H, W, order, B)
    tT, tH, tW = _tile_shape(order, B)
    nT, nH, nW = -(-T // tT), -(-H // tH), -(-W // tW)
    assert perm.size == nT * nH * nW * B
    real = perm[perm >= 0]
    assert np.array_equal(np.sort(real), np.arange(N))
    k = 0
    for a in range(nT):
        for b in range(nH):
            for c in range(nW):
                blk = perm[k * B:(k + 1) * B]
                n = int(blk_len[k])
                assert np.all(blk[:n] >= 0) and np.all(blk[n:] == -1)
                t, y, x = _coords(blk[:n], H, W)
                box = (min(tT, T - a * tT), min(tH, H - b * tH), min(tW, W - c * tW))
                assert n == box[0] * box[1] * box[2]
                assert t.min() == a * tT and y.min() == b * tH and x.min() == c * tW
                assert (np.ptp(t) + 1, np.ptp(y) + 1, np.ptp(x) + 1) == box
                assert np.all(np.diff(blk[:n]) > 0)
                k += 1


@pytest.mark.parametrize("order,shape,B", [("tile2d", (4, 16, 32), 128), ("tile2d", (2, 8, 24), 64),
                                           ("cube3d", (4, 16, 24), 128), ("cube3d", (3, 8, 16), 64)])
def test_tiled_blocks_are_tiles_on_divisible_grids(order, shape, B):
    """When every side is a multiple of the tile, block I is one aligned tile."""
    T, H, W = shape
    perm, blk_len = oracle.plan(T, H, W, order, B)
    assert np.all(blk_len == B)
    tT, tH, tW = _tile_shape(order, B)
    for I in range(perm.size // B):
        t, y, x = _coords(perm[I * B:(I + 1) * B], H, W)
        assert t.min() % tT == 0 and y.min() % tH == 0 and x.min() % tW == 0
        assert (t.max() - t.min(), y.max() - y.min(), x.max() - x.min()) == (tT - 1, tH - 1, tW - 1)


def test_tiled_plans_reduce_to_row_major():
    """One tile per frame (2D) or per grid (3D) gives the row-major order."""
    row, _ = oracle.plan(3, 8, 16, "row", 128)
    assert np.array_equal(oracle.plan(3, 8, 16, "tile2d", 128)[0], row)
    row, _ = oracle.plan(1, 8, 8, "row", 64)
    assert np.array_equal(oracle.plan(1, 8, 8, "cube3d", 64)[0], row)
    assert np.array_equal(oracle.plan(1, 8, 8, "tile2d", 64)[0], row)


def test_tiled_blocks_are_more_compact_than_raster():
    """The 2D and 3D partitions keep blocks as compact boxes on the Wan grid."""
    w = wl.get(3)

    def mean_box(order):
        perm, _ = oracle.plan(w.T, w.H, w.W, order, w.B)
        vols = []
        for I in range(perm.size // w.B):
            t, y, x = _coords(perm[I * w.B:(I + 1) * w.B][perm[I * w.B:(I + 1) * w.B] >= 0], w.H, w.W)
            vols.append((np.ptp(t) + 1) * (np.ptp(y) + 1) * (np.ptp(x) + 1))
        return float(np.mean(vols))

    row = mean_box("row")
    assert mean_box("tile2d") * 2 < row and mean_box("cube3d") * 2 < row


# ---------------------------------------------------------------- 2D Hilbert (per-frame) order

def test_2d_order1_is_gray_code(golden_dir):
    with open(os.path.join(golden_dir, "hilbert2d_order1.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for r in rows:
        idx, y, x = int(r[0]), int(r[2]), int(r[3])
        assert int(oracle.hilbert_index_2d(np.array([y]), np.array([x]), 1)[0]) == idx


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6])
def test_2d_square_bijection_unit_steps_quadrants(b):
    """A bijection onto [0, 4^b) with unit steps; every aligned run of 4^k
    indices fills one aligned 2^k square; starts at (0, 0), ends at (2^b-1, 0)."""
    S = 1 << b
    y, x = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    h = oracle.hilbert_index_2d(y.ravel(), x.ravel(), b)
    assert np.array_equal(np.sort(h), np.arange(S * S))
    order = np.argsort(h)
    yy, xx = y.ravel()[order], x.ravel()[order]
    assert np.all(np.abs(np.diff(yy)) + np.abs(np.diff(xx)) == 1)
    assert (yy[0], xx[0]) == (0, 0) and (yy[-1], xx[-1]) == (S - 1, 0)
    for k in range(1, b):
        run = 1 << (2 * k)
        for s0 in range(0, S * S, run):
            ys, xs = yy[s0:s0 + run], xx[s0:s0 + run]
            assert ys.min() % (1 << k) == 0 and xs.min() % (1 << k) == 0
            assert np.ptp(ys) == (1 << k) - 1 and np.ptp(xs) == (1 << k) - 1


@pytest.mark.parametrize("shape,B", [((3, 5, 7), 64), ((21, 30, 52), 128), ((2, 16, 16), 64), ((1, 1, 1), 64)])
def test_hilbert2d_plan(shape, B):
    """Frame-major; each frame's in-grid cells in the order of the enclosing
    square's curve (brute-force filter of the full square); tail pads."""
    T, H, W = shape
    N = T * H * W
    perm, blk_len = oracle.plan(T, H, W, "hilbert2d", B)
    assert perm.size == -(-N // B) * B and np.all(perm[N:] == -1) and blk_len.sum() == N
    b = max(1, (max(H, W) - 1).bit_length())
    S = 1 << b
    yy, xx = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    cell_at = {int(h): (int(y), int(x)) for h, y, x in
               zip(oracle.hilbert_index_2d(yy.ravel(), xx.ravel(), b), yy.ravel(), xx.ravel())}
    frame = [cell_at[h][0] * W + cell_at[h][1] for h in range(S * S)
             if cell_at[h][0] < H and cell_at[h][1] < W]         # walk the whole square, keep in-grid
    for t in range(T):
        assert np.array_equal(perm[t * H * W:(t + 1) * H * W], t * H * W + np.array(frame))
    t, r = np.divmod(perm[:N], H * W)
    assert np.array_equal(t, np.repeat(np.arange(T), H * W))
