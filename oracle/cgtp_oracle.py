"""fp64 CPU oracle of the Clebsch-Gordan tensor-product (CGTP) convolution, forward and
gradients.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product package, and it imports
nothing from the product.  Plain, slow, obviously correct: numpy fp64, exact
rational arithmetic for the Clebsch-Gordan coefficients, library primitives
(``scipy.special.lpmv``, ``numpy.matmul``, ``numpy.add.reduceat``) as single steps,
no blocking or fusion.

What the pages give, and where (sources are the pages' titles and sections):

* LunaTP, "Enabling Efficient and Scalable Tensor Product for Equivariant MLIPs",
  Abstract: the CGTP convolution is the core cost and the accelerated kernel keeps
  "the underlying mathematical formulation"; Figure 3(a): node-centric execution
  accumulates the edge messages of a receiver before one store; Table 1: the irreps
  cases (hidden irreps x edge irreps -> output irreps) that fix the path rule and the
  channel-wise ("uvu") output multiplicities.
* BranchIP, "Learning Adaptive Equivariant Computation for Interatomic Potentials",
  Method (sparse evaluation; proof intuition): zero-gated features are left out of
  the tensor product, and the sparse result equals the dense one.  Allegro paragraph:
  neighbours are the atoms within a fixed cutoff distance.
* TransIP, "Learning Inter-Atomic Potentials without Explicit Equivariance",
  Sec. 2.1, Eq. (1): the equivariance definition f(phi(g)x) = rho(g) f(x) used by the
  rotation tests.

The pages print no formula for the convolution itself.  The plainest reading, used
here, is the textbook definition: for every active edge j -> i and every path
p = (l1 of an input irrep, l2 of an edge-SH irrep, l3)

    out[i, c_p(u), m3] += w[e, c_p(u)] * sum_{m1,m2} C_p[m1,m2,m3] x[j,u,m1] Y_{l2,m2}(r_ij)

with r_ij = pos[j] - pos[i] + shift_e . cell.  Every other reading taken where the
pages are silent (real basis, phases, normalisation, layouts, edge direction, periodic
minimum image, tie-breaks) is stated at the function that uses it.

Pins (tests/test_oracle_*.py): Table 1 output irreps for all six cases; sympy's exact
CG; orthogonality both ways; stretched and l=1 closed forms; swap symmetry; real-CG
imaginary/real residual exactly 0; real SH closed forms for l <= 2, Unsoeld's theorem,
quadrature orthonormality, rotation covariance; neighbour list against
scipy.spatial.cKDTree and the Si shell count; mask prepare against a second loop;
conv against a pure-Python loop, textbook special cases (SpMV, cross product, dot
product) and SO(3) / inversion / translation / permutation / linearity /
sparse-equals-dense invariants.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from decimal import Decimal, getcontext
from fractions import Fraction
from functools import lru_cache

import numpy as np
import scipy.special

PATHS_ALL = 0
PATHS_PARITY = 1


# --------------------------------------------------------------------------------------
# Irreps and paths.  LunaTP Table 1 ("Irrep configurations used in the kernel
# microbenchmarks"): spec strings "mul x l parity".  The path rule and the uvu
# multiplicity are the readings that reproduce every output irreps string of Table 1.
# --------------------------------------------------------------------------------------

def parse_irreps(spec: str):
    """Parse "128x0e+64x1o" into [(mul, l, parity)], parity +1 for 'e', -1 for 'o'.

    A bare term "1o" means multiplicity 1.  Raises ValueError on malformed input.
    """
    if not isinstance(spec, str) or not spec.strip():
        raise ValueError("empty irreps spec")
    out = []
    for term in spec.replace(" ", "").split("+"):
        if not term:
            raise ValueError(f"empty term in {spec!r}")
        if "x" in term:
            mul_s, ir = term.split("x", 1)
            if not mul_s.isdigit():
                raise ValueError(f"bad multiplicity in {term!r}")
            mul = int(mul_s)
        else:
            mul, ir = 1, term
        if len(ir) < 2 or ir[-1] not in "eo" or not ir[:-1].isdigit():
            raise ValueError(f"bad irrep {term!r}")
        out.append((mul, int(ir[:-1]), 1 if ir[-1] == "e" else -1))
    return out


def format_irreps(irreps) -> str:
    return "+".join(f"{mul}x{l}{'e' if p == 1 else 'o'}" for mul, l, p in irreps)


@dataclass(frozen=True)
class Path:
    l1: int
    p1: int
    l2: int
    p2: int
    l3: int
    p3: int
    mul: int
    i_in: int      # index of the input irrep
    i_sh: int      # index of the edge-SH irrep
    in_off: int    # float offset of the input irrep block in a row of x
    out_off: int   # float offset of this path's block in a row of out
    w_off: int     # first weight column (= first global output channel) of this path


@dataclass(frozen=True)
class Plan:
    irreps_in: tuple
    irreps_sh: tuple
    irreps_out: tuple
    paths: tuple
    f_in: int
    f_out: int
    w_per_edge: int
    l_sh_max: int


def build_plan(irreps_in: str, irreps_sh: str, l_out_max: int, rule: int) -> Plan:
    """Enumerate the uvu paths and the layouts of x, out and w.

    Paths: for each input irrep (spec order), each SH irrep (spec order) and each l3
    from |l1-l2| to min(l1+l2, l_out_max): output parity p1*p2; rule PARITY keeps the
    path only when p1*p2 == (-1)**l3, rule ALL keeps every triangle-allowed path.  Path
    multiplicity = mul of the input irrep (one weight per edge, path and channel).
    Output irreps are sorted by (l3, 'e' before 'o'); inside one output irrep the
    path blocks follow path order.  Reading (layout unpinned by the pages beyond the
    sorted order visible in Table 1): each block is stored [channel][2l+1], and the
    weight column of an output channel equals its global channel index.
    """
    ins = parse_irreps(irreps_in)
    shs = parse_irreps(irreps_sh)
    if rule not in (PATHS_ALL, PATHS_PARITY):
        raise ValueError("unknown path rule")
    for mul, _, _ in shs:
        if mul != 1:
            raise ValueError("edge SH irreps must have multiplicity 1")
    in_offs, off = [], 0
    for mul, l, _ in ins:
        in_offs.append(off)
        off += mul * (2 * l + 1)
    f_in = off

    raw = []
    for i_in, (mul, l1, p1) in enumerate(ins):
        for i_sh, (_, l2, p2) in enumerate(shs):
            for l3 in range(abs(l1 - l2), min(l1 + l2, l_out_max) + 1):
                p3 = p1 * p2
                if rule == PATHS_PARITY and p3 != (-1) ** l3:
                    continue
                raw.append((l1, p1, l2, p2, l3, p3, mul, i_in, i_sh))

    keys = sorted({(r[4], r[5]) for r in raw}, key=lambda k: (k[0], 0 if k[1] == 1 else 1))
    placed = {}
    irreps_out = []
    float_off = 0
    chan_off = 0
    for (l3, p3) in keys:
        members = [k for k, r in enumerate(raw) if (r[4], r[5]) == (l3, p3)]
        c_in_irrep = 0
        for k in members:
            mul = raw[k][6]
            placed[k] = (float_off + c_in_irrep * (2 * l3 + 1), chan_off + c_in_irrep)
            c_in_irrep += mul
        irreps_out.append((c_in_irrep, l3, p3))
        float_off += c_in_irrep * (2 * l3 + 1)
        chan_off += c_in_irrep
    paths = tuple(
        Path(*r, in_off=in_offs[r[7]], out_off=placed[k][0], w_off=placed[k][1])
        for k, r in enumerate(raw)
    )
    return Plan(tuple(ins), tuple(shs), tuple(irreps_out), paths, f_in, float_off,
                chan_off, max(l for _, l, _ in shs))


# --------------------------------------------------------------------------------------
# Clebsch-Gordan coefficients.  Complex CG by Racah's closed form with exact integer
# factorials (one square root at the end), then the change to the real basis.
# Reading (pages silent): Condon-Shortley phase, no path normalisation.
# --------------------------------------------------------------------------------------

getcontext().prec = 60


def cg_complex(j1: int, m1: int, j2: int, m2: int, J: int, M: int) -> float:
    """<j1 m1 j2 m2 | J M> by Racah's formula; exact rational until one sqrt."""
    if M != m1 + m2 or J < abs(j1 - j2) or J > j1 + j2:
        return 0.0
    if abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0.0
    f = math.factorial
    pre = Fraction((2 * J + 1) * f(J + j1 - j2) * f(J - j1 + j2) * f(j1 + j2 - J),
                   f(j1 + j2 + J + 1))
    pre *= f(J + M) * f(J - M) * f(j1 - m1) * f(j1 + m1) * f(j2 - m2) * f(j2 + m2)
    s = Fraction(0)
    for k in range(0, j1 + j2 - J + 1):
        args = (k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k)
        if min(args) < 0:
            continue
        den = 1
        for a in args:
            den *= f(a)
        s += Fraction((-1) ** k, den)
    if s == 0:
        return 0.0
    sq = pre * s * s                     # exact value of the coefficient squared
    mag = (Decimal(sq.numerator) / Decimal(sq.denominator)).sqrt()
    return float(mag) if s > 0 else -float(mag)


def u_matrix(l: int) -> np.ndarray:
    """Unitary map complex SH -> real SH: Y_real[m] = sum_mu U[m, mu] Y_complex[mu].

    Rows m = -l..l (real index), columns mu = -l..l (complex index).  With the
    Condon-Shortley complex SH this gives the real SH of ``real_sh`` below.
    """
    n = 2 * l + 1
    U = np.zeros((n, n), dtype=np.complex128)
    r = 1.0 / math.sqrt(2.0)
    for m in range(-l, l + 1):
        if m < 0:
            U[m + l, m + l] = 1j * r
            U[m + l, -m + l] = -1j * r * (-1) ** m
        elif m == 0:
            U[l, l] = 1.0
        else:
            U[m + l, -m + l] = r
            U[m + l, m + l] = r * (-1) ** m
    return U


@lru_cache(maxsize=None)
def _real_cg_both(l1: int, l2: int, l3: int):
    n1, n2, n3 = 2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1
    C = np.zeros((n1, n2, n3))
    for a in range(-l1, l1 + 1):
        for b in range(-l2, l2 + 1):
            c = a + b
            if abs(c) <= l3:
                C[a + l1, b + l2, c + l3] = cg_complex(l1, a, l2, b, l3, c)
    T = np.einsum("ia,jb,kc,abc->ijk", u_matrix(l1).conj(), u_matrix(l2).conj(),
                  u_matrix(l3), C)
    if (l1 + l2 + l3) % 2 == 0:
        return T.real.copy(), T.imag.copy()
    return T.imag.copy(), T.real.copy()


def real_cg(l1: int, l2: int, l3: int) -> np.ndarray:
    """Real-basis CG tensor C[m1, m2, m3] (fp64), m in -l..l order.

    C = conj(U_l1) (x) conj(U_l2) (x) U_l3 applied to the complex CG; the real part is
    kept when l1+l2+l3 is even and the imaginary part when it is odd (the other part
    vanishes, which ``real_cg_residual`` exposes for the tests).
    """
    return _real_cg_both(l1, l2, l3)[0].copy()


def real_cg_residual(l1: int, l2: int, l3: int) -> float:
    return float(np.abs(_real_cg_both(l1, l2, l3)[1]).max())


# --------------------------------------------------------------------------------------
# Real spherical harmonics.  Reading (pages silent): "component" normalisation,
# sum_m Y_lm^2 = 2l+1 on the unit sphere, Y_00 = 1; the real basis reached by
# ``u_matrix`` from the Condon-Shortley complex SH, so l=1 is sqrt(3)*(y, z, x).
# Computed from associated Legendre functions (scipy.special.lpmv, whose
# Condon-Shortley factor (-1)^m is removed) and trigonometric functions of the polar
# angles.  A zero vector has no direction: Y_0 = 1 and Y_l = 0 for l >= 1.
# --------------------------------------------------------------------------------------

def real_sh(l: int, vec: np.ndarray) -> np.ndarray:
    """Y_l(vec/|vec|) for vec of shape [..., 3]; returns [..., 2l+1] fp64."""
    v = np.asarray(vec, dtype=np.float64)
    shp = v.shape[:-1]
    v = v.reshape(-1, 3)
    r = np.sqrt((v * v).sum(axis=1))
    zero = r == 0.0
    rs = np.where(zero, 1.0, r)
    x, y, z = v[:, 0] / rs, v[:, 1] / rs, v[:, 2] / rs
    ct = np.clip(z, -1.0, 1.0)
    phi = np.arctan2(y, x)
    out = np.zeros((v.shape[0], 2 * l + 1))
    for m in range(0, l + 1):
        p = (-1) ** m * scipy.special.lpmv(m, l, ct)
        if m == 0:
            out[:, l] = math.sqrt(2 * l + 1) * p
        else:
            nrm = math.sqrt(2.0) * math.sqrt((2 * l + 1) * math.factorial(l - m) / math.factorial(l + m))
            out[:, l + m] = nrm * p * np.cos(m * phi)
            out[:, l - m] = nrm * p * np.sin(m * phi)
    if l > 0:
        out[zero] = 0.0
    else:
        out[zero] = 1.0
    return out.reshape(*shp, 2 * l + 1)


def wigner_d_real(l: int, R: np.ndarray, n_points: int = 0, seed: int = 12345) -> np.ndarray:
    """Real Wigner-D of rotation R in the real SH basis, fitted from the SH.

    D is the matrix with Y_l(R r) = D Y_l(r) for all r; it is solved by least squares
    from Y_l at random points and at the rotated points (exact for a representation;
    the tests check D orthogonal and D(R1 R2) = D(R1) D(R2)).
    """
    n = n_points or (4 * (2 * l + 1) + 8)
    P = np.random.default_rng(seed).standard_normal((n, 3))
    Y = real_sh(l, P)
    YR = real_sh(l, P @ np.asarray(R, dtype=np.float64).T)
    Dt, *_ = np.linalg.lstsq(Y, YR, rcond=None)
    return Dt.T


def random_rotation(rng: np.random.Generator) -> np.ndarray:
    """Uniform random rotation from a normalised Gaussian quaternion (uniform on S^3),
    the SO(3) sampling that TransIP's training draws rotations from (Sec. 3.2)."""
    q = rng.standard_normal(4)
    q /= np.linalg.norm(q)
    a, b, c, d = q
    return np.array([
        [a * a + b * b - c * c - d * d, 2 * (b * c - a * d), 2 * (b * d + a * c)],
        [2 * (b * c + a * d), a * a - b * b + c * c - d * d, 2 * (c * d - a * b)],
        [2 * (b * d - a * c), 2 * (c * d + a * b), a * a - b * b - c * c + d * d],
    ])


# --------------------------------------------------------------------------------------
# Neighbour list.  BranchIP (Allegro paragraph): neighbours are the atoms within a
# fixed cutoff distance.  Readings: periodic orthorhombic box under the minimum image
# convention, strict "<", no self edges, rows grouped by receiver i and sorted by
# sender j.  The predicate is evaluated in fp64 in a fixed order so that any
# implementation can reproduce it bit for bit:
#   d = (double)x_j - (double)x_i;  if d > L/2: d -= L, s = -1  elif d < -L/2: d += L, s = +1
#   r2 = (dx*dx + dy*dy) + dz*dz;   edge iff r2 < (double)rc * (double)rc and i != j.
# --------------------------------------------------------------------------------------

def neighbors(pos: np.ndarray, box, cutoff):
    """Brute-force O(N^2) receiver-CSR neighbour list.

    Returns (row_ptr int32 [N+1], col int32 [E], shift int8 [E,3]); the edge r_ij is
    pos[j] - pos[i] + shift . diag(box).
    """
    p = np.asarray(pos, dtype=np.float32).astype(np.float64)
    L = np.asarray(box, dtype=np.float32).astype(np.float64)
    rc = np.float64(np.float32(cutoff))
    rc2 = rc * rc
    n = p.shape[0]
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    cols, shifts = [], []
    jj = np.arange(n)
    for i in range(n):
        d = p - p[i]                       # x_j - x_i per component
        s = np.zeros((n, 3), dtype=np.int8)
        for k in range(3):
            dk = d[:, k]
            half = 0.5 * L[k]
            gt = dk > half
            lt = (~gt) & (dk < -half)
            dk[gt] -= L[k]
            dk[lt] += L[k]
            s[gt, k] = -1
            s[lt, k] = 1
        r2 = (d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2]
        sel = (r2 < rc2) & (jj != i)
        cols.append(jj[sel])
        shifts.append(s[sel])
        row_ptr[i + 1] = row_ptr[i] + int(sel.sum())
    col = np.concatenate(cols).astype(np.int32) if n else np.zeros(0, np.int32)
    shift = np.concatenate(shifts).astype(np.int8) if n else np.zeros((0, 3), np.int8)
    return row_ptr.astype(np.int32), col, shift.reshape(-1, 3)


# --------------------------------------------------------------------------------------
# Mask prepare.  BranchIP (sparse evaluation): edges whose gate is zero are left out
# of the tensor product.  LunaTP Table 9: tasks ordered by node degree, descending
# order being the fastest.  Readings: mask u8, nonzero = active; active edges keep CSR
# order; node order = active degree descending, then node id ascending.
# --------------------------------------------------------------------------------------

def prepare(row_ptr: np.ndarray, mask: np.ndarray | None):
    """Return (act_row_ptr int32 [N+1], act_eid int32 [E_act], order int32 [N])."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    n = row_ptr.shape[0] - 1
    e = int(row_ptr[-1])
    active = np.ones(e, dtype=bool) if mask is None else (np.asarray(mask) != 0)
    act_eid = np.nonzero(active)[0]
    deg = np.array([int(active[row_ptr[i]:row_ptr[i + 1]].sum()) for i in range(n)], dtype=np.int64)
    act_row_ptr = np.zeros(n + 1, dtype=np.int64)
    act_row_ptr[1:] = np.cumsum(deg)
    order = np.array(sorted(range(n), key=lambda i: (-deg[i], i)), dtype=np.int64)
    return act_row_ptr.astype(np.int32), act_eid.astype(np.int32), order.astype(np.int32)


# --------------------------------------------------------------------------------------
# The convolution.  Definition in the module docstring; LunaTP Figure 3(a): messages
# of all incoming edges of a receiver are summed into that receiver.
# --------------------------------------------------------------------------------------

def edge_vectors(pos, cell, row_ptr, col, shift, edge_ids=None):
    """r_ij = pos[j] - pos[i] + shift_e . cell (cell rows are lattice vectors), fp64.

    Reading (pages silent): the edge points from the receiver i to the sender j.
    ``cell`` None means open boundaries (shift ignored)."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    n = row_ptr.shape[0] - 1
    recv = np.repeat(np.arange(n), np.diff(row_ptr))
    ids = np.arange(int(row_ptr[-1])) if edge_ids is None else np.asarray(edge_ids, dtype=np.int64)
    p = np.asarray(pos, dtype=np.float64)
    i = recv[ids]
    j = np.asarray(col, dtype=np.int64)[ids]
    r = p[j] - p[i]
    if cell is not None and shift is not None:
        r = r + np.asarray(shift, dtype=np.float64)[ids] @ np.asarray(cell, dtype=np.float64).reshape(3, 3)
    return r


def edge_sh(plan: Plan, r: np.ndarray) -> np.ndarray:
    """Concatenated real SH of the edge-SH irreps, [E, sum(2 l2 + 1)], fp64."""
    if r.shape[0] == 0:
        return np.zeros((0, sum(2 * l + 1 for _, l, _ in plan.irreps_sh)))
    return np.concatenate([real_sh(l, r) for _, l, _ in plan.irreps_sh], axis=1)


def _active_mask(mask, gate, n_edges):
    """BranchIP sparse evaluation (Method): an edge is active when the mask (if any) keeps
    it and its continuation gate (if any) is not exactly zero."""
    if mask is None and gate is None:
        return None
    act = np.ones(n_edges, dtype=bool)
    if mask is not None:
        act &= np.asarray(mask) != 0
    if gate is not None:
        act &= np.asarray(gate, dtype=np.float64) != 0.0
    return act.astype(np.uint8)


def conv_forward(plan: Plan, pos, cell, row_ptr, col, shift, x, w, mask=None, gate=None) -> np.ndarray:
    """out [N, F_out] fp64.  Inactive edges (mask == 0, or gate == 0) are never read:
    their w and x_j cannot reach the output even when they hold NaN.  Rows with no
    active edge are exactly 0.  gate [E] (optional): BranchIP's continuation gate, which
    multiplies each edge's feature before the tensor product (BranchIP, Method); the
    product is linear in that feature, so the edge's message is scaled by gate[e]."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    n = row_ptr.shape[0] - 1
    act_row_ptr, act_eid, _ = prepare(row_ptr, _active_mask(mask, gate, len(col)))
    act_row_ptr = act_row_ptr.astype(np.int64)
    ids = act_eid.astype(np.int64)
    out = np.zeros((n, plan.f_out))
    if ids.size == 0:
        return out
    r = edge_vectors(pos, cell, row_ptr, col, shift, ids)
    Y = {l: real_sh(l, r) for _, l, _ in plan.irreps_sh}
    recv_rows = np.nonzero(np.diff(act_row_ptr) > 0)[0]
    starts = act_row_ptr[recv_rows]
    j = np.asarray(col, dtype=np.int64)[ids]
    xf = np.asarray(x, dtype=np.float64)
    wf = np.asarray(w, dtype=np.float64)
    for p in plan.paths:
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        C = real_cg(p.l1, p.l2, p.l3)
        xj = xf[j, p.in_off:p.in_off + p.mul * n1].reshape(-1, p.mul, n1)
        A = np.einsum("abc,eb->eac", C, Y[p.l2])          # [E_act, n1, n3]
        msg = np.matmul(xj, A)                            # [E_act, mul, n3]
        msg *= wf[ids, p.w_off:p.w_off + p.mul][:, :, None]
        if gate is not None:
            msg *= np.asarray(gate, dtype=np.float64)[ids][:, None, None]
        summed = np.add.reduceat(msg, starts, axis=0)     # one sum per receiver
        out[recv_rows, p.out_off:p.out_off + p.mul * n3] += summed.reshape(len(recv_rows), -1)
    return out


def conv_forward_loops(plan: Plan, pos, cell, row_ptr, col, shift, x, w, mask=None, gate=None) -> np.ndarray:
    """The same definition as pure-Python loops over receiver, edge, path, channel,
    m1, m2, m3 (for tiny inputs only): the brute-force cross-check of conv_forward."""
    row_ptr = [int(v) for v in row_ptr]
    n = len(row_ptr) - 1
    out = np.zeros((n, plan.f_out))
    cellm = None if cell is None else np.asarray(cell, dtype=np.float64).reshape(3, 3)
    for i in range(n):
        for e in range(row_ptr[i], row_ptr[i + 1]):
            if mask is not None and mask[e] == 0:
                continue
            g = 1.0 if gate is None else float(gate[e])
            if g == 0.0:
                continue
            j = int(col[e])
            r = [float(pos[j][k]) - float(pos[i][k]) for k in range(3)]
            if cellm is not None and shift is not None:
                for k in range(3):
                    r[k] += sum(float(shift[e][a]) * cellm[a][k] for a in range(3))
            for p in plan.paths:
                C = real_cg(p.l1, p.l2, p.l3)
                Y = real_sh(p.l2, np.array(r))
                for u in range(p.mul):
                    wv = float(w[e][p.w_off + u])
                    for m3 in range(2 * p.l3 + 1):
                        acc = 0.0
                        for m1 in range(2 * p.l1 + 1):
                            xv = float(x[j][p.in_off + u * (2 * p.l1 + 1) + m1])
                            for m2 in range(2 * p.l2 + 1):
                                acc += C[m1, m2, m3] * xv * Y[m2]
                        out[i, p.out_off + u * (2 * p.l3 + 1) + m3] += g * wv * acc
    return out


# --------------------------------------------------------------------------------------
# Gradients of the convolution (the backward pass; LunaTP Abstract: its kernels cover the
# derivatives that forces need).  The forward is trilinear in (x_j, w_e, Y(r_e)), so the
# gradients of a scalar L with dL/d out = grad_out are its adjoints, written out:
#   dL/dw[e, c_p(u)]       = g_e sum_{m1,m2,m3} C_p[m1,m2,m3] x[j,u,m1] Y[m2] gout[i,c_p(u),m3]
#   dL/dx[j, u, m1]       += g_e w[e,c_p(u)] sum_{m2,m3} C_p[m1,m2,m3] Y[m2] gout[i,c_p(u),m3]
#   dL/dY_{l2}[e, m2]     += g_e w[e,c_p(u)] sum_{m1,m3} C_p[m1,m2,m3] x[j,u,m1] gout[i,c_p(u),m3]
#   dL/dr_e                = sum_{l2,m2} dL/dY[e, m2] dY_{l2,m2}/dr (r_e)
#   dL/dpos[j] += dL/dr_e,  dL/dpos[i] -= dL/dr_e          (r_e = pos[j] - pos[i] + ...)
# with g_e the continuation gate (1 without one); inactive edges have zero gradients and
# contribute nothing.  The gate, mask, cell and shifts are constants.
# --------------------------------------------------------------------------------------

def real_sh_grad(l: int, vec: np.ndarray) -> np.ndarray:
    """dY_l(vec/|vec|)/d vec for vec of shape [..., 3]; returns [..., 2l+1, 3] fp64.

    Spherical coordinates of real_sh: Y = N P(cos theta) T(m phi) with T = cos or sin, so
    grad Y = (e_theta dY/dtheta + e_phi (1/sin theta) dY/dphi) / |vec|, with
    dP_l^m(cos theta)/dtheta = (l cos theta P_l^m - (l+m) P_{l-1}^m) / sin theta (the
    standard recurrence (x^2 - 1) dP_l^m/dx = l x P_l^m - (l+m) P_{l-1}^m, any fixed
    phase convention) and e_theta = (cos t cos p, cos t sin p, -sin t),
    e_phi = (-sin p, cos p, 0).  Undefined on the z axis (sin theta = 0) and at the
    origin: those raise.  l = 0 has zero gradient."""
    v = np.asarray(vec, dtype=np.float64)
    shp = v.shape[:-1]
    v = v.reshape(-1, 3)
    out = np.zeros((v.shape[0], 2 * l + 1, 3))
    if l == 0 or v.shape[0] == 0:
        return out.reshape(*shp, 2 * l + 1, 3)
    r = np.sqrt((v * v).sum(axis=1))
    rho = np.sqrt(v[:, 0] ** 2 + v[:, 1] ** 2)
    if np.any(r == 0.0) or np.any(rho <= 1e-12 * r):
        raise ValueError("real_sh_grad: a vector is zero or on the z axis")
    ct, st = v[:, 2] / r, rho / r
    phi = np.arctan2(v[:, 1], v[:, 0])
    cp, sp = np.cos(phi), np.sin(phi)
    e_t = np.stack([ct * cp, ct * sp, -st], axis=1)
    e_p = np.stack([-sp, cp, np.zeros_like(sp)], axis=1)
    for m in range(0, l + 1):
        pl = (-1) ** m * scipy.special.lpmv(m, l, ct)
        plm1 = (-1) ** m * scipy.special.lpmv(m, l - 1, ct) if m <= l - 1 else np.zeros_like(ct)
        dpl = (l * ct * pl - (l + m) * plm1) / st            # d P_l^m(cos theta) / d theta
        if m == 0:
            nrm = math.sqrt(2 * l + 1)
            out[:, l, :] = (nrm * dpl)[:, None] * e_t
        else:
            nrm = math.sqrt(2.0) * math.sqrt((2 * l + 1) * math.factorial(l - m) / math.factorial(l + m))
            cm, sm = np.cos(m * phi), np.sin(m * phi)
            # + m: N P cos(m phi);  - m: N P sin(m phi)
            out[:, l + m, :] = (nrm * dpl * cm)[:, None] * e_t + (nrm * pl * (-m * sm) / st)[:, None] * e_p
            out[:, l - m, :] = (nrm * dpl * sm)[:, None] * e_t + (nrm * pl * (m * cm) / st)[:, None] * e_p
    out /= r[:, None, None]
    return out.reshape(*shp, 2 * l + 1, 3)


def conv_backward(plan: Plan, pos, cell, row_ptr, col, shift, x, w, grad_out, mask=None, gate=None):
    """Gradients (grad_x [N, F_in], grad_w [E, W], grad_pos [N, 3]) of a scalar L whose
    gradient with respect to conv_forward's output is grad_out [N, F_out]; fp64.
    Inactive edges get grad_w rows of exactly 0 and their w and x_j are never read."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    n = row_ptr.shape[0] - 1
    e_all = len(col)
    xf = np.asarray(x, dtype=np.float64)
    wf = np.asarray(w, dtype=np.float64)
    gf = np.asarray(grad_out, dtype=np.float64)
    grad_x = np.zeros((n, plan.f_in))
    grad_w = np.zeros((e_all, plan.w_per_edge))
    grad_pos = np.zeros((n, 3))
    _, act_eid, _ = prepare(row_ptr, _active_mask(mask, gate, e_all))
    ids = act_eid.astype(np.int64)
    if ids.size == 0:
        return grad_x, grad_w, grad_pos
    recv = np.repeat(np.arange(n), np.diff(row_ptr))
    i = recv[ids]
    j = np.asarray(col, dtype=np.int64)[ids]
    r = edge_vectors(pos, cell, row_ptr, col, shift, ids)
    g = np.ones(ids.size) if gate is None else np.asarray(gate, dtype=np.float64)[ids]
    Y = {l: real_sh(l, r) for _, l, _ in plan.irreps_sh}
    gY = {l: np.zeros((ids.size, 2 * l + 1)) for _, l, _ in plan.irreps_sh}
    for p in plan.paths:
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        C = real_cg(p.l1, p.l2, p.l3)
        xj = xf[j, p.in_off:p.in_off + p.mul * n1].reshape(-1, p.mul, n1)
        gi = gf[i, p.out_off:p.out_off + p.mul * n3].reshape(-1, p.mul, n3)
        wv = wf[ids, p.w_off:p.w_off + p.mul]
        A = np.einsum("abc,eb->eac", C, Y[p.l2])                       # [E_act, n1, n3]
        t = np.matmul(xj, A)                                            # [E_act, mul, n3]
        grad_w[ids, p.w_off:p.w_off + p.mul] += g[:, None] * (t * gi).sum(axis=2)
        gx = np.einsum("eac,euc->eua", A, gi) * (g[:, None] * wv)[:, :, None]
        np.add.at(grad_x[:, p.in_off:p.in_off + p.mul * n1], j, gx.reshape(ids.size, -1))
        gY[p.l2] += np.einsum("abc,eua,euc,eu->eb", C, xj, gi, g[:, None] * wv)
    grad_r = np.zeros((ids.size, 3))
    for _, l, _ in plan.irreps_sh:
        if l > 0:
            grad_r += np.einsum("eb,ebk->ek", gY[l], real_sh_grad(l, r))
    np.add.at(grad_pos, j, grad_r)
    np.add.at(grad_pos, i, -grad_r)
    return grad_x, grad_w, grad_pos


# --------------------------------------------------------------------------------------
# Cost model of the plain formulation, for reporting only.
# --------------------------------------------------------------------------------------

def cg_nnz(l1: int, l2: int, l3: int) -> int:
    return int((np.abs(real_cg(l1, l2, l3)) > 1e-12).sum())


__all__ = [
    "PATHS_ALL", "PATHS_PARITY", "parse_irreps", "format_irreps", "Path", "Plan",
    "build_plan", "cg_complex", "u_matrix", "real_cg", "real_cg_residual", "real_sh",
    "wigner_d_real", "random_rotation", "neighbors", "prepare", "edge_vectors",
    "edge_sh", "conv_forward", "conv_forward_loops", "real_sh_grad", "conv_backward", "cg_nnz",
]
