"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and places atoms; it holds none of the
convolution's arithmetic, so both the oracle and the HIP path can consume its output
without sharing code.

The workloads stand in for the pages' benchmark systems, whose datasets and trained
models are not available:

* irreps cases from LunaTP Table 1 ("Irrep configurations used in the kernel
  microbenchmarks"), cases 1 and 2, with the 768-atom size of LunaTP Figure 1;
* the silicon diamond lattice (a = 5.43 Angstrom) of LunaTP Figure 6 ("Inference
  scaling"), with a BranchIP-style random per-edge active mask (BranchIP, Method:
  sparse evaluation);
* a 32-atom case small enough for pure-Python loops, and the L_max = 6,
  64-channels-per-degree case of LunaTP Figure 1.

Recipe (every config, seed 0, ``numpy.random.default_rng``), in draw order:
  1. positions: uniform in a cubic box of side L = (N / 0.05)^(1/3) (0.05 atoms per
     cubic Angstrom), drawn in fp64 then cast to fp32; or the diamond lattice plus
     N(0, 0.05 Angstrom) jitter per coordinate, wrapped into [0, L), cast to fp32.
     A coordinate that rounds to L in fp32 is set to 0, so every coordinate is in
     [0, L).
  2. (the neighbour list of the positions fixes the edge count E)
  3. x ~ N(0, 1) [N, F_in] fp32
  4. w ~ N(0, 1) [E, W] fp32
  5. mask (masked configs only): Bernoulli(0.5) per edge in CSR order, uint8.
  6. gate (gated configs only): BranchIP continuation gate per edge in CSR order,
     u = U[0,1), v = U[0,1) drawn as two arrays in that order, gate = 0 where u < 0.5
     (a flat exact-zero region for half the edges) and 1 - v in (0, 1] elsewhere; fp32.

LunaTP Table 1 cases 4-6 (the larger multiplicities and L = 4) are also available at the
768-atom size as c4_768, c5_768 and c6_768.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DENSITY = 0.05          # atoms per cubic Angstrom
SI_LATTICE = 5.43       # Angstrom
SI_JITTER = 0.05        # Angstrom, standard deviation per Cartesian coordinate

RULE_ALL = 0
RULE_PARITY = 1


@dataclass(frozen=True)
class Workload:
    name: str
    n_atoms: int
    cutoff: float
    irreps_in: str
    irreps_sh: str
    l_out_max: int
    rule: int
    lattice: str          # "random" or "si"
    masked: bool
    seed: int = 0
    description: str = ""
    gated: bool = False


def _sh(lmax: int, natural: bool = True) -> str:
    return "+".join(f"1x{l}{('e' if l % 2 == 0 else 'o') if natural else 'e'}" for l in range(lmax + 1))


WORKLOADS = {
    "tiny": Workload(
        "tiny", 32, 4.0, "8x0e+8x1o", _sh(1), 1, RULE_ALL, "random", False,
        description="32 random atoms, cutoff 4 A, 8x0e+8x1o x SH l<=1, all paths l3<=1"),
    "c1_768": Workload(
        "c1_768", 768, 5.0, "128x0e+64x1e+32x2e", _sh(2, natural=False), 2, RULE_ALL, "random", False,
        description="768 random atoms, cutoff 5 A, LunaTP Table 1 case 1 irreps"),
    "c2_768": Workload(
        "c2_768", 768, 5.0, "128x0e+128x1o+128x2e", _sh(3), 3, RULE_PARITY, "random", False,
        description="768 random atoms, cutoff 5 A, LunaTP Table 1 case 2 irreps"),
    "highl_768": Workload(
        "highl_768", 768, 5.0, "+".join(f"64x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(7)),
        _sh(6), 6, RULE_PARITY, "random", False,
        description="768 random atoms, cutoff 5 A, 64 channels per degree l=0..6, SH l<=6"),
    "si_mask": Workload(
        "si_mask", 4096, 5.0, "128x0e+64x1o+32x2e+32x3o", _sh(3), 3, RULE_PARITY, "si", True,
        description="Si diamond 8x8x8 cells (4096 atoms), cutoff 5 A, Bernoulli(0.5) edge mask"),
    "si_gate": Workload(
        "si_gate", 4096, 5.0, "128x0e+64x1o+32x2e+32x3o", _sh(3), 3, RULE_PARITY, "si", False,
        description="Si diamond 8x8x8 cells (4096 atoms), cutoff 5 A, continuous BranchIP gate "
                    "(half the edges exactly 0, the rest in (0, 1])", gated=True),
    "c4_768": Workload(
        "c4_768", 768, 5.0, "256x0e+256x1o+256x2e+256x3o", _sh(3), 3, RULE_PARITY, "random", False,
        description="768 random atoms, cutoff 5 A, LunaTP Table 1 case 4 irreps"),
    "c5_768": Workload(
        "c5_768", 768, 5.0, "320x0e+96x1o+64x2e+32x3o+32x4e", _sh(4), 4, RULE_PARITY, "random", False,
        description="768 random atoms, cutoff 5 A, LunaTP Table 1 case 5 irreps"),
    "c6_768": Workload(
        "c6_768", 768, 5.0, "128x0e+128x1o+128x2e+128x3o+128x4e", _sh(4), 4, RULE_PARITY, "random", False,
        description="768 random atoms, cutoff 5 A, LunaTP Table 1 case 6 irreps"),
}

# configuration order of the benchmark list: tiny, case-1 style, case-2 style, high-L, Si+mask
ORDER = ["tiny", "c1_768", "c2_768", "highl_768", "si_mask"]


def box_length(wl: Workload) -> float:
    if wl.lattice == "si":
        return 8 * SI_LATTICE
    return (wl.n_atoms / DENSITY) ** (1.0 / 3.0)


def _diamond_cells(ncell: int, a: float) -> np.ndarray:
    basis = np.array([
        [0.0, 0.0, 0.0], [0.0, 0.5, 0.5], [0.5, 0.0, 0.5], [0.5, 0.5, 0.0],
        [0.25, 0.25, 0.25], [0.25, 0.75, 0.75], [0.75, 0.25, 0.75], [0.75, 0.75, 0.25],
    ])
    g = np.arange(ncell)
    cells = np.stack(np.meshgrid(g, g, g, indexing="ij"), axis=-1).reshape(-1, 3)
    return ((cells[:, None, :] + basis[None, :, :]) * a).reshape(-1, 3)


def positions(wl: Workload):
    """Draw step 1.  Returns (pos fp32 [N,3], box fp32 [3], cell fp32 [3,3], rng)."""
    rng = np.random.default_rng(wl.seed)
    L = box_length(wl)
    if wl.lattice == "si":
        ideal = _diamond_cells(8, SI_LATTICE)
        assert ideal.shape[0] == wl.n_atoms
        p = np.mod(ideal + rng.normal(0.0, SI_JITTER, ideal.shape), L)
    else:
        p = rng.random((wl.n_atoms, 3)) * L
    box = np.full(3, L, dtype=np.float32)
    p32 = p.astype(np.float32)
    p32[p32 >= box[0]] = 0.0
    cell = np.diag(box).astype(np.float32)
    return p32, box, cell, rng


def features(rng: np.random.Generator, n: int, f_in: int) -> np.ndarray:
    """Draw step 3."""
    return rng.standard_normal((n, f_in)).astype(np.float32)


def weights(rng: np.random.Generator, n_edges: int, w_per_edge: int) -> np.ndarray:
    """Draw step 4."""
    return rng.standard_normal((n_edges, w_per_edge)).astype(np.float32)


def edge_mask(rng: np.random.Generator, n_edges: int) -> np.ndarray:
    """Draw step 5."""
    return (rng.random(n_edges) < 0.5).astype(np.uint8)


def gate_values(wl: Workload, rng: np.random.Generator, n_edges: int):
    """Draw step 6 (after draw_payload): the continuation gate of a gated config, else None."""
    if not wl.gated:
        return None
    u = rng.random(n_edges)
    v = rng.random(n_edges)
    return np.where(u < 0.5, 0.0, 1.0 - v).astype(np.float32)


def draw_payload(wl: Workload, rng: np.random.Generator, n_atoms: int, f_in: int,
                 n_edges: int, w_per_edge: int):
    """Steps 3-5 in order.  Returns (x, w, mask or None)."""
    x = features(rng, n_atoms, f_in)
    w = weights(rng, n_edges, w_per_edge)
    mask = edge_mask(rng, n_edges) if wl.masked else None
    return x, w, mask
