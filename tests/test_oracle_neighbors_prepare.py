"""Pins of the oracle's neighbour list and mask prepare.

Independent references: scipy.spatial.cKDTree with periodic box (a library routine),
pair symmetry, the shell structure of the diamond lattice, and a second pure-Python
implementation of the prepare step.
"""
import numpy as np
import pytest
from scipy.spatial import cKDTree

import oracle as O
import workloads as WL


def _pairs(row_ptr, col):
    n = len(row_ptr) - 1
    recv = np.repeat(np.arange(n), np.diff(row_ptr))
    return set(zip(recv.tolist(), col.tolist()))


@pytest.mark.parametrize("name", ["tiny", "c1_768", "si_mask"])
def test_neighbors_vs_kdtree(name):
    wl = WL.WORKLOADS[name]
    pos, box, cell, _ = WL.positions(wl)
    row_ptr, col, shift = O.neighbors(pos, box, wl.cutoff)
    assert row_ptr[0] == 0 and row_ptr[-1] == len(col) == len(shift)
    assert np.all(pos >= 0) and np.all(pos < box[0])
    # scipy's periodic KD-tree (pairs i<j with distance <= r): compare the sets
    tree = cKDTree(pos.astype(np.float64), boxsize=box.astype(np.float64))
    ref = tree.query_pairs(float(np.float32(wl.cutoff)), output_type="ndarray")
    ref_set = set(map(tuple, ref.tolist())) | set(map(tuple, ref[:, ::-1].tolist()))
    got = _pairs(row_ptr, col)
    # ties at exactly the cutoff are measure-zero; the strict and non-strict tests agree
    assert got == ref_set
    # rows sorted by j, no self edges
    for i in range(len(row_ptr) - 1):
        seg = col[row_ptr[i]:row_ptr[i + 1]]
        assert np.all(np.diff(seg) > 0) and not np.any(seg == i)
    # shifts reproduce a vector shorter than the cutoff, and are antisymmetric
    r = O.edge_vectors(pos, cell, row_ptr, col, shift)
    assert np.all(np.linalg.norm(r, axis=1) < wl.cutoff)
    recv = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    lookup = {(int(recv[e]), int(col[e])): shift[e] for e in range(len(col))}
    for (i, j), s in lookup.items():
        assert np.array_equal(lookup[(j, i)], -s)


def test_mean_degrees_and_si_shells():
    for name, lo, hi in [("tiny", 11.0, 15.0), ("c1_768", 24.5, 27.5)]:
        wl = WL.WORKLOADS[name]
        pos, box, _, _ = WL.positions(wl)
        row_ptr, _, _ = O.neighbors(pos, box, wl.cutoff)
        assert lo < row_ptr[-1] / wl.n_atoms < hi
    wl = WL.WORKLOADS["si_mask"]
    pos, box, _, _ = WL.positions(wl)
    row_ptr, _, _ = O.neighbors(pos, box, wl.cutoff)
    deg = np.diff(row_ptr)
    # diamond shells: 4 at a*sqrt(3)/4, 12 at a/sqrt(2), 12 at a*sqrt(11)/4 (< 5 A),
    # next 6 at a = 5.43 A (> 5 A)
    assert deg.min() == deg.max() == 28 and row_ptr[-1] == 114688


def test_predicate_is_strict_and_bitwise():
    # two atoms exactly at the cutoff along x: no edge; one ulp closer: edge
    box = np.full(3, 20.0, dtype=np.float32)
    pos = np.array([[1.0, 1.0, 1.0], [5.0, 1.0, 1.0]], dtype=np.float32)
    rp, col, _ = O.neighbors(pos, box, 4.0)
    assert rp[-1] == 0
    pos[1, 0] = np.nextafter(np.float32(5.0), np.float32(0.0))
    rp, col, sh = O.neighbors(pos, box, 4.0)
    assert rp.tolist() == [0, 1, 2] and col.tolist() == [1, 0]
    # minimum image across the boundary
    pos = np.array([[0.5, 1.0, 1.0], [19.0, 1.0, 1.0]], dtype=np.float32)
    rp, col, sh = O.neighbors(pos, box, 4.0)
    # r_01 = x_1 - x_0 + s L = 18.5 - 20: the image one box to the left
    assert col.tolist() == [1, 0] and sh.tolist() == [[-1, 0, 0], [1, 0, 0]]


def _prepare_loops(row_ptr, mask):
    n = len(row_ptr) - 1
    act_ptr, eids, deg = [0], [], []
    for i in range(n):
        d = 0
        for e in range(row_ptr[i], row_ptr[i + 1]):
            if mask is None or mask[e]:
                eids.append(e)
                d += 1
        deg.append(d)
        act_ptr.append(act_ptr[-1] + d)
    order = []
    for d in range(max(deg, default=0), -1, -1):      # degree descending, id ascending
        order += [i for i in range(n) if deg[i] == d]
    return act_ptr, eids, order


@pytest.mark.parametrize("seed", range(4))
def test_prepare_vs_loops(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 60))
    deg = rng.integers(0, 9, n)
    row_ptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    mask = (rng.random(int(row_ptr[-1])) < 0.5).astype(np.uint8) if seed % 2 else None
    a, e, o = O.prepare(row_ptr, mask)
    ra, re_, ro = _prepare_loops(row_ptr.tolist(), None if mask is None else mask.tolist())
    assert a.tolist() == ra and e.tolist() == re_ and o.tolist() == ro
