"""MI355X-native Clebsch-Gordan tensor-product (CGTP) convolution, forward (fp32; fp64 for l <= 4).

Thin binding over libcgtp.so (C ABI in include/cgtp.h): argument marshalling only.
Every step of the path (neighbour list, mask prepare, edge harmonics, the fused
convolution) runs in the library's HIP kernels on the caller's current torch stream;
torch provides device memory and streams.  There is no CPU fallback: without the
built library or a gfx950 device the calls raise.

    plan = Plan("128x0e+128x1o+128x2e", "1x0e+1x1o+1x2e+1x3o", 3, "parity")
    row_ptr, col, shift = neighbors_build(pos, box, cutoff)
    out = conv_forward(plan, pos, cell, row_ptr, col, shift, x, w, mask)
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import CGTP_PATHS_ALL, CGTP_PATHS_PARITY, CgtpError, check, load

__all__ = ["Plan", "neighbors_build", "conv_prepare", "edge_sh", "conv_forward", "conv_backward", "CgtpError",
           "CGTP_PATHS_ALL", "CGTP_PATHS_PARITY", "library_path", "version"]


def library_path() -> str:
    return _lib.LIB_PATH


def version() -> str:
    return load().cgtp_version().decode()


def _rule(rule) -> int:
    if isinstance(rule, str):
        return {"all": CGTP_PATHS_ALL, "parity": CGTP_PATHS_PARITY}[rule]
    return int(rule)


class Plan:
    """A CGTP plan: irreps, paths, real-CG tables and the wave-job schedule."""

    def __init__(self, irreps_in: str, irreps_sh: str, l_out_max: int, path_rule="parity",
                 host_only: bool = False, fp64: bool = False):
        lib = load()
        h = ctypes.c_void_p()
        flags = (_lib.CGTP_PLAN_HOST_ONLY if host_only else 0) | (_lib.CGTP_PLAN_FP64 if fp64 else 0)
        check(lib.cgtp_plan_create(irreps_in.encode(), irreps_sh.encode(), int(l_out_max),
                                   _rule(path_rule), flags, ctypes.byref(h)))
        self._h = h
        f_in, f_out, w = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        npaths, lsh = ctypes.c_int(), ctypes.c_int()
        buf = ctypes.create_string_buffer(4096)
        check(lib.cgtp_plan_info(h, ctypes.byref(f_in), ctypes.byref(f_out), ctypes.byref(w),
                                 ctypes.byref(npaths), ctypes.byref(lsh), buf, 4096))
        self.f_in, self.f_out, self.w_per_edge = f_in.value, f_out.value, w.value
        self.n_paths, self.l_sh_max = npaths.value, lsh.value
        self.sh_stride = (self.l_sh_max + 1) ** 2
        self.irreps_out = buf.value.decode()
        self.host_only = host_only
        self.fp64 = fp64
        self.dtype = torch.float64 if fp64 else torch.float32

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan is closed")
        return self._h

    def paths(self) -> np.ndarray:
        """[n_paths, 10] int32: l1, p1, l2, p2, l3, p3, mul, in_off, out_off, w_off."""
        rows = np.zeros((self.n_paths, 10), dtype=np.int32)
        check(load().cgtp_plan_paths(self.handle, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return rows

    def cg(self, path: int) -> np.ndarray:
        l1, _, l2, _, l3 = (int(v) for v in self.paths()[path][:5])
        out = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1), dtype=np.float32)
        check(load().cgtp_plan_cg(self.handle, int(path), out.ctypes.data_as(_lib.FP)))
        return out

    def schedule(self):
        nj, nv = ctypes.c_int(), ctypes.c_int()
        check(load().cgtp_plan_schedule(self.handle, ctypes.byref(nj), ctypes.byref(nv)))
        return nj.value, nv.value

    def workspace_size(self, n_nodes: int, n_edges: int, has_mask: bool = False) -> int:
        b = ctypes.c_size_t()
        check(load().cgtp_workspace_size(self.handle, int(n_nodes), int(n_edges), int(bool(has_mask)),
                                         ctypes.byref(b)))
        return b.value

    def backward_workspace_size(self, n_nodes: int, n_edges: int) -> int:
        b = ctypes.c_size_t()
        check(load().cgtp_backward_workspace_size(self.handle, int(n_nodes), int(n_edges), ctypes.byref(b)))
        return b.value

    def close(self):
        if getattr(self, "_h", None) is not None:
            load().cgtp_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _dev(t: torch.Tensor, dtype, name: str, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device (cuda) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _host_f32(v, n, name):
    if v is None:
        return None
    a = np.ascontiguousarray(np.asarray(v.cpu() if isinstance(v, torch.Tensor) else v, dtype=np.float32).reshape(-1))
    if a.size != n:
        raise ValueError(f"{name} must have {n} values")
    return a


def _host_f64(v, n, name):
    if v is None:
        return None
    a = np.ascontiguousarray(np.asarray(v.cpu() if isinstance(v, torch.Tensor) else v, dtype=np.float64).reshape(-1))
    if a.size != n:
        raise ValueError(f"{name} must have {n} values")
    return a


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def neighbors_build(pos: torch.Tensor, box, cutoff: float, edge_capacity: int | None = None):
    """Receiver-CSR neighbour list under the minimum image convention (synchronises).

    Returns (row_ptr int32 [N+1], col int32 [E], shift int8 [E,3])."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    n = pos.shape[0]
    boxa = _host_f32(box, 3, "box")
    bp = boxa.ctypes.data_as(_lib.FP)
    wsb = ctypes.c_size_t()
    check(lib.cgtp_neighbors_workspace_size(n, bp, float(cutoff), ctypes.byref(wsb)))
    ws = torch.empty(max(wsb.value, 256), dtype=torch.uint8, device=pos.device)
    row_ptr = torch.empty(n + 1, dtype=torch.int32, device=pos.device)
    cap = int(edge_capacity) if edge_capacity is not None else max(64, 48 * n)
    for _ in range(2):
        col = torch.empty(max(cap, 1), dtype=torch.int32, device=pos.device)
        shift = torch.empty((max(cap, 1), 3), dtype=torch.int8, device=pos.device)
        ne = ctypes.c_int64()
        rc = lib.cgtp_neighbors_build(_ptr(pos), n, bp, float(cutoff), _ptr(row_ptr), _ptr(col), _ptr(shift),
                                      cap, ctypes.byref(ne), _ptr(ws), ws.numel(), _stream())
        if rc == _lib.CGTP_ERR_CAPACITY:
            cap = ne.value
            continue
        check(rc)
        e = ne.value
        return row_ptr, col[:e], shift[:e]
    raise CgtpError(_lib.CGTP_ERR_CAPACITY, "edge capacity retry failed")


def conv_prepare(plan: Plan, row_ptr: torch.Tensor, mask: torch.Tensor | None, n_edges: int, workspace=None):
    """Active CSR and node order.  Returns (act_row_ptr [N+1], act_eid [n_edges] (the
    first act_row_ptr[N] entries are valid), order [N])."""
    lib = load()
    _dev(row_ptr, torch.int32, "row_ptr")
    n = row_ptr.shape[0] - 1
    if mask is not None:
        _dev(mask, torch.uint8, "mask", (n_edges,))
    dev = row_ptr.device
    act_row_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
    act_eid = torch.empty(max(n_edges, 1), dtype=torch.int32, device=dev)
    order = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    ws = _workspace(plan.workspace_size(n, n_edges, mask is not None), dev, workspace)
    check(lib.cgtp_conv_prepare(plan.handle, _ptr(row_ptr), _ptr(mask), n, n_edges, _ptr(act_row_ptr),
                                _ptr(act_eid), _ptr(order), _ptr(ws), ws.numel(), _stream()))
    return act_row_ptr, act_eid[:n_edges], order[:n]


def edge_sh(plan: Plan, pos, cell, row_ptr, col, shift):
    """Real SH of every edge, [E, (l_sh_max+1)^2] fp32 (block l at offset l*l)."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    _dev(row_ptr, torch.int32, "row_ptr")
    _dev(col, torch.int32, "col")
    n, e = pos.shape[0], col.shape[0]
    if shift is not None:
        _dev(shift, torch.int8, "shift", (e, 3))
    cella = _host_f32(cell, 9, "cell")
    sh = torch.empty((max(e, 1), plan.sh_stride), dtype=torch.float32, device=pos.device)
    check(lib.cgtp_edge_sh(plan.handle, _ptr(pos), n, None if cella is None else cella.ctypes.data_as(_lib.FP),
                           _ptr(row_ptr), _ptr(col), _ptr(shift), e, _ptr(sh), _stream()))
    return sh[:e]


def conv_forward(plan: Plan, pos, cell, row_ptr, col, shift, x, w, mask=None, out=None, workspace=None,
                 conv_events=None, gate=None):
    """out[N, f_out] of the CGTP convolution (asynchronous on the current stream).

    gate: optional [E] continuation gate (BranchIP): zero-gated edges are inactive,
    the others' messages are scaled by the gate.
    conv_events: optional (begin, end) torch.cuda.Event pair (each recorded once before,
    so that its HIP event exists); the library records them around the fused
    convolution kernel launches.
    pos, x, w, gate and out are fp32, or fp64 for a plan made with fp64=True."""
    lib = load()
    dt = plan.dtype
    _dev(pos, dt, "pos")
    n = pos.shape[0]
    _dev(row_ptr, torch.int32, "row_ptr", (n + 1,))
    _dev(col, torch.int32, "col")
    e = col.shape[0]
    if shift is not None:
        _dev(shift, torch.int8, "shift", (e, 3))
    _dev(x, dt, "x", (n, plan.f_in))
    _dev(w, dt, "w", (e, plan.w_per_edge))
    if mask is not None:
        _dev(mask, torch.uint8, "mask", (e,))
    if gate is not None:
        _dev(gate, dt, "gate", (e,))
    if out is None:
        out = torch.empty((n, plan.f_out), dtype=dt, device=pos.device)
    _dev(out, dt, "out", (n, plan.f_out))
    ws = _workspace(plan.workspace_size(n, e, mask is not None), pos.device, workspace)
    if plan.fp64:
        cella = _host_f64(cell, 9, "cell")
        ev = (None, None) if conv_events is None else tuple(ctypes.c_void_p(v.cuda_event) for v in conv_events)
        check(lib.cgtp_conv_forward_f64(
            plan.handle, _ptr(pos), n, None if cella is None else cella.ctypes.data_as(_lib.DP),
            _ptr(row_ptr), _ptr(col), _ptr(shift), e, _ptr(x), _ptr(w), _ptr(mask), _ptr(gate),
            _ptr(out), _ptr(ws), ws.numel(), _stream(), ev[0], ev[1]))
        return out
    cella = _host_f32(cell, 9, "cell")
    args = (plan.handle, _ptr(pos), n, None if cella is None else cella.ctypes.data_as(_lib.FP),
            _ptr(row_ptr), _ptr(col), _ptr(shift), e, _ptr(x), _ptr(w), _ptr(mask), _ptr(gate),
            _ptr(out), _ptr(ws), ws.numel(), _stream())
    if conv_events is None:
        check(lib.cgtp_conv_forward_gated(*args))
    else:
        b, t = conv_events
        check(lib.cgtp_conv_forward_timed(*args, ctypes.c_void_p(b.cuda_event), ctypes.c_void_p(t.cuda_event)))
    return out


def conv_backward(plan: Plan, pos, cell, row_ptr, col, shift, x, w, grad_out, mask=None, gate=None,
                  need=("x", "w", "pos"), workspace=None):
    """Gradients of a scalar L with dL/d out = grad_out [N, f_out] (fp32, l <= 4 plans):
    returns (grad_x [N, f_in], grad_w [E, W], grad_pos [N, 3]); an entry not in `need`
    is None.  Asynchronous on the current stream."""
    lib = load()
    _dev(pos, torch.float32, "pos")
    n = pos.shape[0]
    _dev(row_ptr, torch.int32, "row_ptr", (n + 1,))
    _dev(col, torch.int32, "col")
    e = col.shape[0]
    if shift is not None:
        _dev(shift, torch.int8, "shift", (e, 3))
    _dev(x, torch.float32, "x", (n, plan.f_in))
    _dev(w, torch.float32, "w", (e, plan.w_per_edge))
    _dev(grad_out, torch.float32, "grad_out", (n, plan.f_out))
    if mask is not None:
        _dev(mask, torch.uint8, "mask", (e,))
    if gate is not None:
        _dev(gate, torch.float32, "gate", (e,))
    dev = pos.device
    gx = torch.empty((n, plan.f_in), dtype=torch.float32, device=dev) if "x" in need else None
    gw = torch.empty((e, plan.w_per_edge), dtype=torch.float32, device=dev) if "w" in need else None
    gp = torch.empty((n, 3), dtype=torch.float32, device=dev) if "pos" in need else None
    ws = _workspace(plan.backward_workspace_size(n, e), dev, workspace)
    cella = _host_f32(cell, 9, "cell")
    check(lib.cgtp_conv_backward(plan.handle, _ptr(pos), n, None if cella is None else cella.ctypes.data_as(_lib.FP),
                                 _ptr(row_ptr), _ptr(col), _ptr(shift), e, _ptr(x), _ptr(w), _ptr(mask), _ptr(gate),
                                 _ptr(grad_out), _ptr(gx), _ptr(gw), _ptr(gp), _ptr(ws), ws.numel(), _stream()))
    return gx, gw, gp
