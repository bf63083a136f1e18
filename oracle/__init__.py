"""fp64 CPU oracle for the 2-D TM Maxwell FDTD propagator (ctypes binding).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product package.
It shares no code with the GPU path; both consume the seeded arrays of
``tm_maxwell_fdtd_amd.inputs`` (the oracle receives the float32-rounded
values widened back to float64, see ``inputs.as_f32``).

The arithmetic lives in ``tm_oracle.c`` (plain C, fp64, OpenMP over rows);
this module only marshals arrays.  Every function's definition and the
page passages it follows are documented in that file.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tm_oracle.c")
_LIB = os.path.join(_HERE, "liborac.so")

_ll = ctypes.c_longlong
_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_longlong)


class Geom(ctypes.Structure):
    _fields_ = [
        ("order", ctypes.c_int),
        ("periodic", ctypes.c_int),
        ("n_shots", _ll), ("ny", _ll), ("nx", _ll),
        ("pml_y0", _ll), ("pml_y1", _ll), ("pml_x0", _ll), ("pml_x1", _ll),
        ("rdy", ctypes.c_double), ("rdx", ctypes.c_double),
        ("n_src", _ll), ("n_rec", _ll),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liborac.so``."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.orc_forward.restype = ctypes.c_int
        L.orc_forward.argtypes = [ctypes.POINTER(Geom), _dp, _dp, _dp, _dp, _ll, _dp, _lp, _lp,
                                  _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ll, _ll, _ll]
        L.orc_adjoint_range.restype = ctypes.c_int
        L.orc_adjoint_range.argtypes = [ctypes.POINTER(Geom), _dp, _dp, _dp, _dp, _ll, _lp, _lp, _dp, _dp,
                                        _dp, _dp, _ll, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ll, _ll]
        L.orc_adjoint.restype = ctypes.c_int
        L.orc_adjoint.argtypes = [ctypes.POINTER(Geom), _dp, _dp, _dp, _dp, _ll, _lp, _lp, _ll,
                                  _dp, _dp, _dp, _dp, _dp, _dp]
        L.orc_shot_sum.restype = None
        L.orc_shot_sum.argtypes = [_ll, _ll, _dp, _dp]
        L.orc_eps_sigma_grad.restype = None
        L.orc_eps_sigma_grad.argtypes = [_ll, _dp, _dp, ctypes.c_double, _dp, _dp, _dp, _dp]
        L.orc_e4m3_encode.restype = ctypes.c_int
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_int]
        L.orc_quantize_e4m3.restype = None
        L.orc_quantize_e4m3.argtypes = [_ll, _dp]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_num_threads.argtypes = []
        L.orc_coefficients.restype = ctypes.c_int
        L.orc_coefficients.argtypes = [ctypes.c_int, _dp]
        _lib = L
    return _lib


def _d(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.cast(None, _dp)
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_dp)


def _l(a: np.ndarray):
    assert a.dtype == np.int64 and a.flags.c_contiguous
    return a.ctypes.data_as(_lp)


def _c64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def geom(wl, periodic: bool = False) -> Geom:
    return Geom(order=wl.order, periodic=int(periodic), n_shots=wl.n_shots, ny=wl.ny, nx=wl.nx,
                pml_y0=wl.pml_y0, pml_y1=wl.pml_y1, pml_x0=wl.pml_x0, pml_x1=wl.pml_x1,
                rdy=1.0 / wl.dy, rdx=1.0 / wl.dx, n_src=wl.n_src, n_rec=wl.n_rec)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


def coefficients(order: int) -> np.ndarray:
    c = np.zeros(4)
    n = lib().orc_coefficients(order, _d(c))
    if n < 0:
        raise ValueError(f"order {order} not supported")
    return c[:n]


class State:
    """Forward state of all shots: fields and the four CPML memories."""

    def __init__(self, n_shots, ny, nx):
        shape = (n_shots, ny, nx)
        self.E = np.zeros(shape)
        self.Hx = np.zeros(shape)
        self.Hz = np.zeros(shape)
        self.psi_ez = np.zeros(shape)
        self.psi_ex = np.zeros(shape)
        self.psi_hxz = np.zeros(shape)
        self.psi_hzx = np.zeros(shape)

    def copy(self):
        out = State.__new__(State)
        for k, v in self.__dict__.items():
            setattr(out, k, v.copy())
        return out


def forward(wl, t0: int = 0, t1: Optional[int] = None, state: Optional[State] = None,
            store: bool = False, periodic: bool = False, ca=None, cb=None, cq=None, f=None,
            segment: bool = False, records: Optional[np.ndarray] = None):
    """Run forward steps t0..t1-1.  Returns (records, state, snapshots).

    ``records`` is [nt][S][n_rec] (rows outside [t0, t1) are zero, or keep
    what a passed-in ``records`` array held);
    ``snapshots`` is None or a pair (Ey^n, curlH^n) of [nt][S][ny_i][nx_i]
    (with ``segment``: of [t1 - t0][S][ny_i][nx_i], step n at n - t0).
    ``ca``/``cb``/``cq``/``f`` override the workload's arrays.
    """
    t1 = wl.nt if t1 is None else t1
    g = geom(wl, periodic)
    st = State(wl.n_shots, wl.ny, wl.nx) if state is None else state
    r = np.zeros((wl.nt, wl.n_shots, wl.n_rec)) if records is None else records
    assert r.shape == (wl.nt, wl.n_shots, wl.n_rec) and r.dtype == np.float64 and r.flags.c_contiguous
    snaps = None
    snap_t0 = t0 if segment else 0
    if store:
        nyi, nxi = wl.pml_y1 - wl.pml_y0, wl.pml_x1 - wl.pml_x0
        steps = (t1 - t0) if segment else wl.nt
        snaps = (np.zeros((steps, wl.n_shots, nyi, nxi)), np.zeros((steps, wl.n_shots, nyi, nxi)))
    ca = _c64(wl.ca if ca is None else ca)
    cb = _c64(wl.cb if cb is None else cb)
    cq = _c64(wl.cq if cq is None else cq)
    f = _c64(wl.f if f is None else f)
    cpml = _c64(wl.cpml)
    src = np.ascontiguousarray(wl.src, dtype=np.int64)
    rec = np.ascontiguousarray(wl.rec, dtype=np.int64)
    rc = lib().orc_forward(ctypes.byref(g), _d(ca), _d(cb), _d(cq), _d(cpml), cpml.shape[1],
                           _d(f), _l(src), _l(rec), _d(st.E), _d(st.Hx), _d(st.Hz),
                           _d(st.psi_ez), _d(st.psi_ex), _d(st.psi_hxz), _d(st.psi_hzx),
                           _d(r), _d(snaps[0] if snaps else None), _d(snaps[1] if snaps else None),
                           snap_t0, t0, t1)
    if rc != 0:
        raise RuntimeError(f"orc_forward failed ({rc})")
    return r, st, snaps


def adjoint(wl, grad_r: np.ndarray, snaps=None, ca=None, cb=None, cq=None, want_grad_f=True):
    """Exact adjoint.  Returns (grad_f [nt][S][n_src], gca [S][ny][nx], gcb [S][ny][nx])."""
    g = geom(wl)
    grad_r = _c64(grad_r)
    assert grad_r.shape == (wl.nt, wl.n_shots, wl.n_rec)
    grad_f = np.zeros((wl.nt, wl.n_shots, wl.n_src)) if want_grad_f else None
    gca = np.zeros((wl.n_shots, wl.ny, wl.nx))
    gcb = np.zeros((wl.n_shots, wl.ny, wl.nx))
    ca = _c64(wl.ca if ca is None else ca)
    cb = _c64(wl.cb if cb is None else cb)
    cq = _c64(wl.cq if cq is None else cq)
    cpml = _c64(wl.cpml)
    src = np.ascontiguousarray(wl.src, dtype=np.int64)
    rec = np.ascontiguousarray(wl.rec, dtype=np.int64)
    se = _c64(snaps[0]) if snaps is not None else None
    sc = _c64(snaps[1]) if snaps is not None else None
    rc = lib().orc_adjoint(ctypes.byref(g), _d(ca), _d(cb), _d(cq), _d(cpml), cpml.shape[1],
                           _l(src), _l(rec), wl.nt, _d(grad_r), _d(grad_f), _d(se), _d(sc),
                           _d(gca), _d(gcb))
    if rc != 0:
        raise RuntimeError(f"orc_adjoint failed ({rc})")
    return grad_f, gca, gcb


class AdjointState:
    """Adjoint state of all shots: lambda_E, lambda_Hx, lambda_Hz and the
    adjoint memories of the four CPML filters (zero before step nt-1)."""

    NAMES = ("lE", "lHx", "lHz", "m_hzx", "m_hxz", "m_ex", "m_ez")

    def __init__(self, n_shots, ny, nx):
        for k in self.NAMES:
            setattr(self, k, np.zeros((n_shots, ny, nx)))


def adjoint_range(wl, grad_r: np.ndarray, t0: int, t1: int, state: AdjointState, snaps=None,
                  snap_t0: int = 0, gca=None, gcb=None, grad_f=None, ca=None, cb=None, cq=None):
    """Adjoint steps t1-1 .. t0 on ``state`` (updated in place).  ``snaps``
    holds step n at index n - snap_t0; the per-shot gradients are
    accumulated into ``gca`` / ``gcb`` ([S][ny][nx] fp64, may be None) and
    rows t0..t1-1 of ``grad_f`` ([nt][S][n_src], may be None) written."""
    g = geom(wl)
    grad_r = _c64(grad_r)
    assert grad_r.shape == (wl.nt, wl.n_shots, wl.n_rec)
    ca = _c64(wl.ca if ca is None else ca)
    cb = _c64(wl.cb if cb is None else cb)
    cq = _c64(wl.cq if cq is None else cq)
    cpml = _c64(wl.cpml)
    src = np.ascontiguousarray(wl.src, dtype=np.int64)
    rec = np.ascontiguousarray(wl.rec, dtype=np.int64)
    se = _c64(snaps[0]) if snaps is not None else None
    sc = _c64(snaps[1]) if snaps is not None else None
    rc = lib().orc_adjoint_range(ctypes.byref(g), _d(ca), _d(cb), _d(cq), _d(cpml), cpml.shape[1],
                                 _l(src), _l(rec), _d(grad_r), _d(grad_f), _d(se), _d(sc), snap_t0,
                                 *(_d(getattr(state, k)) for k in AdjointState.NAMES),
                                 _d(gca), _d(gcb), t0, t1)
    if rc != 0:
        raise RuntimeError(f"orc_adjoint_range failed ({rc})")


def gradient_checkpointed(wl, every: int, grad_r=None, residual=None, want_grad_f=True, progress=None):
    """Records and the exact adjoint's gradients with bounded memory: the
    forward keeps its state every ``every`` steps; the adjoint replays each
    segment from its checkpoint (storing that segment's snapshots only) and
    runs the segment's reverse steps, last segment first.  The arithmetic is
    that of forward + adjoint (the replay repeats the same steps), so the
    results equal the full-storage ones.

    dJ/dr is ``grad_r`` if given, else ``residual(records)``, else the
    records themselves (J = 1/2 |r|^2).  ``progress(msg)``, if given, is
    called after each forward and adjoint segment.  Returns a dict like
    ``misfit_and_gradient`` (without J)."""
    nt, S = wl.nt, wl.n_shots
    st = State(S, wl.ny, wl.nx)
    r = np.zeros((nt, S, wl.n_rec))
    ckpts = {}
    for ta in range(0, nt, every):
        ckpts[ta] = st.copy()
        forward(wl, ta, min(ta + every, nt), state=st, records=r)
        if progress is not None:
            progress(f"oracle forward {min(ta + every, nt)}/{nt}")
    del st
    if grad_r is None:
        grad_r = r if residual is None else residual(r)
    grad_r = _c64(grad_r)
    adj = AdjointState(S, wl.ny, wl.nx)
    gca = np.zeros((S, wl.ny, wl.nx))
    gcb = np.zeros((S, wl.ny, wl.nx))
    grad_f = np.zeros((nt, S, wl.n_src)) if want_grad_f else None
    for ta in sorted(ckpts, reverse=True):
        tb = min(ta + every, nt)
        _, _, snaps = forward(wl, ta, tb, state=ckpts.pop(ta), store=True, segment=True)
        adjoint_range(wl, grad_r, ta, tb, adj, snaps, snap_t0=ta, gca=gca, gcb=gcb, grad_f=grad_f)
        del snaps
        if progress is not None:
            progress(f"oracle adjoint {ta}/{nt}")
    return dict(records=r, grad_f=grad_f, gca_shot=gca, gcb_shot=gcb, gca=shot_sum(gca), gcb=shot_sum(gcb),
                residual=grad_r)


def shot_sum(grad_shot: np.ndarray) -> np.ndarray:
    gs = _c64(grad_shot)
    out = np.zeros(gs.shape[1:])
    lib().orc_shot_sum(gs.shape[0], int(np.prod(gs.shape[1:])), _d(gs), _d(out))
    return out


def eps_sigma_grad(eps_r, sigma, dt, grad_ca, grad_cb):
    """dJ/deps_r and dJ/dsigma from dJ/dCa and dJ/dCb (chain rule through the
    coefficient definitions, see ``orc_eps_sigma_grad``).  Shapes are kept."""
    eps_r = _c64(eps_r)
    sigma = _c64(sigma)
    gca = _c64(grad_ca)
    gcb = _c64(grad_cb)
    assert eps_r.shape == sigma.shape == gca.shape == gcb.shape
    ge = np.zeros(eps_r.shape)
    gs = np.zeros(eps_r.shape)
    lib().orc_eps_sigma_grad(eps_r.size, _d(eps_r), _d(sigma), float(dt), _d(gca), _d(gcb), _d(ge), _d(gs))
    return ge, gs


def e4m3_encode(x: float) -> int:
    """FP8 E4M3 code of x (round to nearest even, saturating at +-448)."""
    return int(lib().orc_e4m3_encode(float(x)))


def e4m3_decode(code: int) -> float:
    return float(lib().orc_e4m3_decode(int(code)))


def quantize_e4m3(a: np.ndarray) -> np.ndarray:
    """Values an FP8 E4M3 snapshot store keeps for ``a`` (a new fp64 array)."""
    out = np.array(a, dtype=np.float64, order="C", copy=True)
    lib().orc_quantize_e4m3(out.size, _d(out))
    return out


def subsample_snapshots(snaps, step_ratio: int):
    """Snapshots as a store that keeps every ``step_ratio``-th step sees them:
    the kept steps (t % step_ratio == 0) weighted by step_ratio, the others
    zero, so the adjoint's gradient becomes
    sum over kept t of step_ratio * lambda^{t+1} * snapshot^t."""
    out = []
    for a in snaps:
        b = np.zeros_like(a)
        b[::step_ratio] = a[::step_ratio] * float(step_ratio)
        out.append(b)
    return tuple(out)


def misfit_and_gradient(wl, observed=None, snap_quant=None, step_ratio=1):
    """J = 1/2 ||r - d||^2 (d = 0 when ``observed`` is None) and its gradients.

    ``snap_quant="fp8"`` quantizes the stored snapshots to FP8 E4M3 before the
    adjoint uses them (what an FP8 snapshot store keeps); ``step_ratio`` > 1
    keeps every step_ratio-th snapshot only (``subsample_snapshots``).
    Returns dict with records, J, grad_f, per-shot gca/gcb and the shot sums.
    """
    r, _, snaps = forward(wl, store=True)
    if snap_quant == "fp8":
        snaps = (quantize_e4m3(snaps[0]), quantize_e4m3(snaps[1]))
    elif snap_quant is not None:
        raise ValueError(f"unknown snapshot quantization {snap_quant!r}")
    if step_ratio > 1:
        snaps = subsample_snapshots(snaps, step_ratio)
    resid = r if observed is None else r - observed
    J = 0.5 * float(np.sum(resid * resid))
    grad_f, gca, gcb = adjoint(wl, resid, snaps)
    return dict(records=r, J=J, grad_f=grad_f, gca_shot=gca, gcb_shot=gcb,
                gca=shot_sum(gca), gcb=shot_sum(gcb), residual=resid)
