"""ctypes binding of ``libtm_fdtd.so`` (the C ABI in ``include/tm_fdtd.h``).

The functions keep the C names and argument order; they only marshal
arguments (torch tensors become device pointers, the torch stream becomes a
hipStream_t).  Every step of the propagator runs in the library's kernels.
If the library is missing this module raises on load; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtm_fdtd.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "tm_fdtd.h")

TM_OK, TM_EINVAL, TM_EUNSTABLE, TM_ENOMEM, TM_EHIP, TM_ESTATE, TM_ENONFINITE = range(7)
TM_SNAP_F32, TM_SNAP_BF16, TM_SNAP_FP8 = 0, 1, 2
SNAP_KINDS = {"f32": TM_SNAP_F32, "bf16": TM_SNAP_BF16, "fp8": TM_SNAP_FP8}
TM_STORE_DEVICE, TM_STORE_HOST = 0, 1
TM_FWD_STORE, TM_FWD_CHECK = 1, 2

_STATUS_NAMES = {0: "TM_OK", 1: "TM_EINVAL", 2: "TM_EUNSTABLE", 3: "TM_ENOMEM", 4: "TM_EHIP",
                 5: "TM_ESTATE", 6: "TM_ENONFINITE"}


class TmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS_NAMES.get(status, status)} ({status_string(status)})")


class tm_desc(ctypes.Structure):
    _fields_ = [
        ("order", ctypes.c_int32),
        ("snap", ctypes.c_int32),
        ("n_shots", ctypes.c_int64),
        ("ny", ctypes.c_int64), ("nx", ctypes.c_int64),
        ("pml_y0", ctypes.c_int64), ("pml_y1", ctypes.c_int64),
        ("pml_x0", ctypes.c_int64), ("pml_x1", ctypes.c_int64),
        ("dy", ctypes.c_double), ("dx", ctypes.c_double),
        ("nt", ctypes.c_int64),
        ("n_src", ctypes.c_int64), ("n_rec", ctypes.c_int64),
        ("ckpt_every", ctypes.c_int64),
        ("hbm_budget", ctypes.c_uint64),
        ("time_block", ctypes.c_int32),
        ("storage", ctypes.c_int32),
        ("step_ratio", ctypes.c_int64),
        ("model_per_shot", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_vp = ctypes.c_void_p
_lib = None


def lib():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with tm_maxwell_fdtd_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.tm_status_string.restype = ctypes.c_char_p
        L.tm_status_string.argtypes = [ctypes.c_int]
        L.tm_plan_create.restype = ctypes.c_int
        L.tm_plan_create.argtypes = [ctypes.POINTER(tm_desc), _vp, _vp, _vp, ctypes.POINTER(_vp)]
        L.tm_plan_destroy.restype = None
        L.tm_plan_destroy.argtypes = [_vp]
        L.tm_workspace_bytes.restype = ctypes.c_int
        L.tm_workspace_bytes.argtypes = [_vp, ctypes.POINTER(ctypes.c_uint64)]
        L.tm_courant.restype = ctypes.c_int
        L.tm_courant.argtypes = [_vp, _vp, ctypes.c_uint64, _vp, _vp, _vp, ctypes.POINTER(ctypes.c_double)]
        L.tm_courant_noalloc.restype = ctypes.c_int
        L.tm_courant_noalloc.argtypes = [_vp, _vp, _vp, _vp, ctypes.POINTER(ctypes.c_double)]
        L.tm_plan_set_indices.restype = ctypes.c_int
        L.tm_plan_set_indices.argtypes = [_vp, _vp, _vp]
        L.tm_forward.restype = ctypes.c_int
        L.tm_forward.argtypes = [_vp, _vp, ctypes.c_uint64, _vp, _vp, _vp, _vp, _vp,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _vp]
        L.tm_adjoint.restype = ctypes.c_int
        L.tm_adjoint.argtypes = [_vp, _vp, ctypes.c_uint64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.tm_grad.restype = ctypes.c_int
        L.tm_grad.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp]
        L.tm_fp8_encode.restype = ctypes.c_int
        L.tm_fp8_encode.argtypes = [_vp, _vp, ctypes.c_int64, _vp]
        L.tm_fp8_decode.restype = ctypes.c_int
        L.tm_fp8_decode.argtypes = [_vp, _vp, ctypes.c_int64, _vp]
        L.tm_grad_eps_sigma.restype = ctypes.c_int
        L.tm_grad_eps_sigma.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_double, _vp, _vp, _vp]
        L.tm_timing_enable.restype = ctypes.c_int
        L.tm_timing_enable.argtypes = [_vp, ctypes.c_int32]
        L.tm_timing_read.restype = ctypes.c_int
        L.tm_timing_read.argtypes = [_vp, _vp, _vp]
        L.tm_kernel_count.restype = ctypes.c_int32
        L.tm_kernel_count.argtypes = []
        L.tm_kernel_name.restype = ctypes.c_char_p
        L.tm_kernel_name.argtypes = [ctypes.c_int32]
        _lib = L
    return _lib


def declared_functions():
    """Names of the functions ``include/tm_fdtd.h`` declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tm_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().tm_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != TM_OK:
        raise TmError(status, where)


# ---- pointer helpers --------------------------------------------------------

def ptr(t) -> Optional[int]:
    """Device (or host) address of a torch tensor / numpy array, None for None."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        assert t.flags.c_contiguous
        return t.ctypes.data
    assert t.is_contiguous(), "tensors passed to the library must be contiguous"
    return t.data_ptr()


def stream_handle(stream=None) -> Optional[int]:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


# ---- C ABI, same names ------------------------------------------------------

def tm_plan_create(desc: tm_desc, cpml: np.ndarray, src: Optional[np.ndarray], rec: Optional[np.ndarray]):
    cpml = np.ascontiguousarray(cpml, dtype=np.float32)
    src = None if src is None else np.ascontiguousarray(src, dtype=np.int64)
    rec = None if rec is None else np.ascontiguousarray(rec, dtype=np.int64)
    out = _vp()
    st = lib().tm_plan_create(ctypes.byref(desc), ptr(cpml), ptr(src), ptr(rec), ctypes.byref(out))
    return st, out.value


def tm_plan_set_indices(plan, src: Optional[np.ndarray], rec: Optional[np.ndarray]) -> int:
    src = None if src is None else np.ascontiguousarray(src, dtype=np.int64)
    rec = None if rec is None else np.ascontiguousarray(rec, dtype=np.int64)
    return lib().tm_plan_set_indices(plan, ptr(src), ptr(rec))


def tm_plan_destroy(plan):
    lib().tm_plan_destroy(plan)


def tm_workspace_bytes(plan):
    n = ctypes.c_uint64(0)
    st = lib().tm_workspace_bytes(plan, ctypes.byref(n))
    return st, n.value


def tm_courant(plan, ws, ws_bytes, cb, cq, stream):
    c = ctypes.c_double(0.0)
    st = lib().tm_courant(plan, ws, ws_bytes, cb, cq, stream, ctypes.byref(c))
    return st, c.value


def tm_courant_noalloc(plan, cb, cq, stream):
    c = ctypes.c_double(0.0)
    st = lib().tm_courant_noalloc(plan, cb, cq, stream, ctypes.byref(c))
    return st, c.value


def tm_forward(plan, ws, ws_bytes, ca, cb, cq, f, r, t0, t1, flags, stream):
    return lib().tm_forward(plan, ws, ws_bytes, ca, cb, cq, f, r, t0, t1, flags, stream)


def tm_adjoint(plan, ws, ws_bytes, ca, cb, cq, f, grad_r, grad_f, grad_ca_shot, grad_cb_shot, stream):
    return lib().tm_adjoint(plan, ws, ws_bytes, ca, cb, cq, f, grad_r, grad_f, grad_ca_shot,
                            grad_cb_shot, stream)


def tm_grad(plan, grad_ca_shot, grad_cb_shot, grad_ca, grad_cb, stream):
    return lib().tm_grad(plan, grad_ca_shot, grad_cb_shot, grad_ca, grad_cb, stream)


def tm_fp8_encode(inp, out, n, stream):
    return lib().tm_fp8_encode(inp, out, n, stream)


def tm_fp8_decode(inp, out, n, stream):
    return lib().tm_fp8_decode(inp, out, n, stream)


def tm_grad_eps_sigma(plan, ca, cb, grad_ca, grad_cb, dt, grad_eps_r, grad_sigma, stream):
    return lib().tm_grad_eps_sigma(plan, ca, cb, grad_ca, grad_cb, dt, grad_eps_r, grad_sigma, stream)


def tm_status_string(status: int) -> str:
    return status_string(status)


def tm_timing_enable(plan, every: int):
    return lib().tm_timing_enable(plan, int(every))


def tm_kernel_count() -> int:
    return int(lib().tm_kernel_count())


def tm_kernel_name(k: int) -> Optional[str]:
    n = lib().tm_kernel_name(int(k))
    return None if n is None else n.decode()


def tm_timing_read(plan):
    """Returns (status, {kernel name: (total ms, samples)})."""
    n = tm_kernel_count()
    ms = np.zeros(n, dtype=np.float64)
    cnt = np.zeros(n, dtype=np.int64)
    st = lib().tm_timing_read(plan, ms.ctypes.data, cnt.ctypes.data)
    return st, {tm_kernel_name(k): (float(ms[k]), int(cnt[k])) for k in range(n)}


# ---- convenience layer (still marshalling only) -----------------------------

def make_desc(wl, snap: Optional[str] = None, ckpt_every: Optional[int] = None, hbm_budget: int = 0,
              time_block: int = 0, storage: int = 0, step_ratio: int = 0) -> tm_desc:
    snap = wl.snap if snap is None else snap
    per_shot = np.ndim(wl.ca) == 3        # [S][ny][nx]: one model per shot
    return tm_desc(order=wl.order, snap=SNAP_KINDS[snap], model_per_shot=int(per_shot),
                   n_shots=wl.n_shots, ny=wl.ny, nx=wl.nx,
                   pml_y0=wl.pml_y0, pml_y1=wl.pml_y1, pml_x0=wl.pml_x0, pml_x1=wl.pml_x1,
                   dy=wl.dy, dx=wl.dx, nt=wl.nt, n_src=wl.n_src, n_rec=wl.n_rec,
                   ckpt_every=wl.ckpt_every if ckpt_every is None else ckpt_every,
                   hbm_budget=hbm_budget, time_block=time_block, storage=storage, step_ratio=step_ratio)


class Propagator:
    """A plan plus its torch-allocated workspace on one device.

    ``forward``/``adjoint``/``grad`` call the C ABI on the current torch
    stream.  Inputs must be contiguous float32 (int64 for indices) device
    tensors; the model arrays are passed at construction.
    """

    def __init__(self, wl, device="cuda", snap=None, ckpt_every=None, hbm_budget=0, time_block=0, storage=0,
                 step_ratio=0):
        import torch

        self.wl = wl
        self.device = torch.device(device)
        self.desc = make_desc(wl, snap, ckpt_every, hbm_budget, time_block, storage, step_ratio)
        st, plan = tm_plan_create(self.desc, wl.cpml, wl.src, wl.rec)
        _check(st, "tm_plan_create")
        self.plan = plan
        st, nbytes = tm_workspace_bytes(plan)
        _check(st, "tm_workspace_bytes")
        self.ws_bytes = nbytes
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        f32 = dict(dtype=torch.float32, device=self.device)
        self.ca = torch.as_tensor(np.ascontiguousarray(wl.ca, np.float32)).to(**f32)
        self.cb = torch.as_tensor(np.ascontiguousarray(wl.cb, np.float32)).to(**f32)
        self.cq = torch.as_tensor(np.ascontiguousarray(wl.cq, np.float32)).to(**f32)
        self.f = torch.as_tensor(np.ascontiguousarray(wl.f, np.float32)).to(**f32)

    def close(self):
        if getattr(self, "plan", None):
            import torch

            torch.cuda.synchronize(self.device)
            tm_plan_destroy(self.plan)
            self.plan = None
        self.ws = None            # the workspace goes back to torch's allocator

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_indices(self, src, rec):
        """New source / receiver cells ([S][n_src], [S][n_rec] int64) for the
        same plan; the workspace is reallocated when its size changes."""
        import torch

        torch.cuda.synchronize(self.device)
        st = tm_plan_set_indices(self.plan, src, rec)
        _check(st, "tm_plan_set_indices")
        st, nbytes = tm_workspace_bytes(self.plan)
        _check(st, "tm_workspace_bytes")
        if nbytes != self.ws_bytes:
            self.ws = None
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self.ws_bytes = nbytes
        import dataclasses

        self.wl = dataclasses.replace(self.wl, src=np.asarray(src, np.int64), rec=np.asarray(rec, np.int64))

    def courant(self):
        st, c = tm_courant(self.plan, ptr(self.ws), self.ws_bytes, ptr(self.cb), ptr(self.cq),
                           stream_handle())
        _check(st, "tm_courant")
        return c

    def forward(self, r=None, store=False, check=True, t0=0, t1=None):
        import torch

        wl = self.wl
        t1 = wl.nt if t1 is None else t1
        if r is None:
            r = torch.zeros((wl.nt, wl.n_shots, wl.n_rec), dtype=torch.float32, device=self.device)
        flags = (TM_FWD_STORE if store else 0) | (TM_FWD_CHECK if check else 0)
        st = tm_forward(self.plan, ptr(self.ws), self.ws_bytes, ptr(self.ca), ptr(self.cb), ptr(self.cq),
                        ptr(self.f), ptr(r), t0, t1, flags, stream_handle())
        _check(st, "tm_forward")
        return r

    def adjoint(self, grad_r, want_grad_f=True, want_grads=True):
        import torch

        wl = self.wl
        f32 = dict(dtype=torch.float32, device=self.device)
        grad_f = torch.empty((wl.nt, wl.n_shots, wl.n_src), **f32) if want_grad_f else None
        gca = torch.empty((wl.n_shots, wl.ny, wl.nx), **f32) if want_grads else None
        gcb = torch.empty((wl.n_shots, wl.ny, wl.nx), **f32) if want_grads else None
        st = tm_adjoint(self.plan, ptr(self.ws), self.ws_bytes, ptr(self.ca), ptr(self.cb), ptr(self.cq),
                        ptr(self.f), ptr(grad_r.contiguous()), ptr(grad_f), ptr(gca), ptr(gcb),
                        stream_handle())
        _check(st, "tm_adjoint")
        return grad_f, gca, gcb

    def grad(self, gca_shot, gcb_shot):
        import torch

        wl = self.wl
        f32 = dict(dtype=torch.float32, device=self.device)
        gca = torch.empty((wl.ny, wl.nx), **f32) if gca_shot is not None else None
        gcb = torch.empty((wl.ny, wl.nx), **f32) if gcb_shot is not None else None
        st = tm_grad(self.plan, ptr(gca_shot), ptr(gcb_shot), ptr(gca), ptr(gcb), stream_handle())
        _check(st, "tm_grad")
        return gca, gcb

    def grad_eps_sigma(self, gca, gcb, dt=None):
        """dJ/deps_r, dJ/dsigma [ny][nx] from dJ/dCa, dJ/dCb [ny][nx] (either
        may be None) at this propagator's coefficients; ``dt`` defaults to the
        workload's time step.  With one model per shot the inputs and outputs
        are the per-shot [S][ny][nx] arrays, each shot at its own model."""
        import torch

        wl = self.wl
        dt = wl.dt if dt is None else dt
        f32 = dict(dtype=torch.float32, device=self.device)
        per_shot = self.desc.model_per_shot == 1
        shape = (wl.n_shots, wl.ny, wl.nx) if per_shot else (wl.ny, wl.nx)
        geps = torch.empty(shape, **f32)
        gsig = torch.empty(shape, **f32)
        pick = (lambda t, s: None if t is None else t[s]) if per_shot else (lambda t, s: t)
        for s in range(wl.n_shots if per_shot else 1):
            st = tm_grad_eps_sigma(self.plan, ptr(pick(self.ca, s)), ptr(pick(self.cb, s)), ptr(pick(gca, s)),
                                   ptr(pick(gcb, s)), float(dt), ptr(pick(geps, s)), ptr(pick(gsig, s)),
                                   stream_handle())
            _check(st, "tm_grad_eps_sigma")
        return geps, gsig
