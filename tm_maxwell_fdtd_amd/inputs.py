"""Seeded synthetic inputs for the 2-D TM Maxwell FDTD propagator.

This module builds everything a run consumes: the padded grid geometry,
the material model (eps_r, sigma, mu_r), the update coefficients Ca, Cb, Cq,
the CPML profile arrays, the Ricker source wavelet and the source/receiver
cell indices.  It performs none of the propagator's arithmetic (no stencil,
no time step, no adjoint), so the GPU path and the fp64 CPU oracle can both
consume its arrays without sharing any code of the method itself.

Readings of points the source pages leave open (tide-GPR 0.0.9,
``tide/csrc/maxwell.cu``; only its CUDA kernels are on the page, the Python
layer that builds these arrays is not):

* Ca, Cb from eps and sigma: the semi-implicit lossy forms whose derivatives
  are exactly the ones printed in ``convert_grad_ca_cb_to_eps_sigma``
  (dCa/deps = (1-Ca)Cb/dt, dCb/deps = -Cb^2/dt, dCa/dsigma = -(1+Ca)Cb/2,
  dCb/dsigma = -Cb^2/2), with eps = EP0 * eps_r and EP0 as defined there.
  Cq = dt / (mu0 mu_r) is the plain Yee reading.  The 1/dx factors are
  applied inside the stencils (the ``rdx``/``rdy`` constants of the kernels).
* CPML profile: standard convolutional PML with a quadratic damping profile,
  alpha decreasing linearly into the band and kappa = 1 by default (or
  kappa rising quadratically from 1 to ``kappa_max``); integer-grid arrays
  (ax, bx, kx) serve the E-update derivatives and half-grid arrays (axh, ...)
  the H-update derivatives, as in ``forward_kernel_h``/``forward_kernel_e``.
* Ricker wavelet of unit amplitude, delayed by 1.5 periods.
* Time step at 0.9 of the staggered scheme's stability limit.
* Sources on interior row 2, receivers on interior row 5, evenly spread
  along x.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

# Vacuum permittivity as defined by the propagator source (EP0 macro).
EP0 = 8.8541878128e-12
MU0 = 1.25663706212e-6
C0 = 1.0 / math.sqrt(EP0 * MU0)

# Sum of |c_k| of the staggered Taylor coefficients per order.  Only used to
# pick dt at a fixed fraction of the stability limit (an input choice).
_ABS_COEF_SUM = {
    2: 1.0,
    4: 9.0 / 8.0 + 1.0 / 24.0,
    8: 1225.0 / 1024.0 + 245.0 / 3072.0 + 49.0 / 5120.0 + 5.0 / 7168.0,
}

ORDERS = (2, 4, 8)


@dataclasses.dataclass
class Workload:
    """All inputs of one propagation problem, in float64.

    Layout conventions (shared with the C ABI):
      * fields and models are row-major [ny][nx] (x fastest), one [ny][nx]
        slab per shot;
      * ``src`` is [S][n_src] and ``rec`` is [S][n_rec] int64 flat cell
        indices y*nx + x, a negative value meaning "none";
      * ``f`` (source amplitudes) is time-major [nt][S][n_src];
      * ``cpml`` is [12][max(ny, nx)] in the order
        ay, by, ky, ayh, byh, kyh (length ny) then ax, bx, kx, axh, bxh, kxh
        (length nx); rows shorter than the row length are zero-padded.
    """

    name: str
    order: int
    n_shots: int
    ny: int
    nx: int
    pml_y0: int
    pml_y1: int
    pml_x0: int
    pml_x1: int
    dy: float
    dx: float
    dt: float
    nt: int
    eps_r: np.ndarray
    sigma: np.ndarray
    mu_r: np.ndarray
    ca: np.ndarray
    cb: np.ndarray
    cq: np.ndarray
    cpml: np.ndarray
    f: np.ndarray
    src: np.ndarray
    rec: np.ndarray
    freq: float
    snap: str = "f32"          # snapshot storage type on the GPU path
    ckpt_every: int = 0        # 0 = store every step; K > 0 = checkpoint/replay
    obs_eps_r: Optional[np.ndarray] = None   # "observed" model (config 1 misfit)
    extra: Dict[str, object] = dataclasses.field(default_factory=dict)

    @property
    def n_src(self) -> int:
        return int(self.src.shape[1])

    @property
    def n_rec(self) -> int:
        return int(self.rec.shape[1])

    @property
    def half_order(self) -> int:
        return self.order // 2

    @property
    def n_int_y(self) -> int:
        return self.pml_y1 - self.pml_y0

    @property
    def n_int_x(self) -> int:
        return self.pml_x1 - self.pml_x0

    def cell_updates(self) -> int:
        """Cell-updates of one pass: shots x (interior + CPML cells) x steps."""
        p = self.half_order
        return self.n_shots * (self.ny - 2 * p) * (self.nx - 2 * p) * self.nt


# ---------------------------------------------------------------------------
# Building blocks
# ---------------------------------------------------------------------------

def update_coefficients(eps_r, sigma, mu_r, dt):
    """Ca, Cb, Cq (float64) from relative permittivity, conductivity, mu_r."""
    eps = EP0 * np.asarray(eps_r, dtype=np.float64)
    loss = np.asarray(sigma, dtype=np.float64) * dt / (2.0 * eps)
    ca = (1.0 - loss) / (1.0 + loss)
    cb = (dt / eps) / (1.0 + loss)
    cq = dt / (MU0 * np.asarray(mu_r, dtype=np.float64))
    return ca, cb, cq


def stable_dt(eps_r_min, mu_r_min, dy, dx, order, fraction=0.9):
    """dt at ``fraction`` of the stability limit of the staggered scheme."""
    vmax = C0 / math.sqrt(eps_r_min * mu_r_min)
    return fraction / (vmax * _ABS_COEF_SUM[order] * math.sqrt(1.0 / dx ** 2 + 1.0 / dy ** 2))


def cpml_axis(n, lo, hi, npml, h, dt, vmax, freq, r_coef=1e-3, kappa_max=1.0):
    """CPML profile arrays for one axis of ``n`` points.

    ``lo`` is the first interior index and ``hi`` one past the last one.
    Returns (a, b, k, ah, bh, kh), each of length n, for integer points
    (x) and half points (x + 1/2 stored at x).  Outside the band the
    damping is zero (a = 0) and kappa = 1, so a kernel that ignored its band
    flag would still not damp there.  Inside the band kappa grows as
    1 + (kappa_max - 1) xi^2 with the normalised depth xi, like the damping.
    """
    if npml <= 0:
        z = np.zeros(n)
        one = np.ones(n)
        return z, z.copy(), one, z.copy(), z.copy(), one.copy()
    width = npml * h
    d0 = -3.0 * vmax * math.log(r_coef) / (2.0 * width)
    alpha0 = math.pi * freq

    def profile(pos):
        xi = np.zeros_like(pos)
        left = pos < lo
        right = pos > hi - 1
        xi[left] = (lo - pos[left]) / npml
        xi[right] = (pos[right] - (hi - 1)) / npml
        xi = np.clip(xi, 0.0, None)
        d = d0 * xi ** 2
        alpha = alpha0 * np.clip(1.0 - xi, 0.0, None)
        kappa = 1.0 + (kappa_max - 1.0) * xi ** 2
        b = np.exp(-(d / kappa + alpha) * dt)
        denom = kappa * (d + kappa * alpha)
        a = np.where(d > 0.0, d * (b - 1.0) / np.where(denom > 0.0, denom, 1.0), 0.0)
        return a, b, kappa

    idx = np.arange(n, dtype=np.float64)
    a, b, k = profile(idx)
    ah, bh, kh = profile(idx + 0.5)
    return a, b, k, ah, bh, kh


def pack_cpml(ny, nx, y_arrays, x_arrays):
    """Pack the 12 profile arrays into the [12][max(ny, nx)] layout."""
    m = max(ny, nx)
    out = np.zeros((12, m), dtype=np.float64)
    for i, arr in enumerate(y_arrays):
        out[i, :ny] = arr
    for i, arr in enumerate(x_arrays):
        out[6 + i, :nx] = arr
    return out


def identity_cpml(ny, nx):
    """Profile with a = b = 0 and kappa = 1: the CPML filter is the identity."""
    z_y, z_x = np.zeros(ny), np.zeros(nx)
    return pack_cpml(ny, nx, (z_y, z_y, np.ones(ny), z_y, z_y, np.ones(ny)),
                     (z_x, z_x, np.ones(nx), z_x, z_x, np.ones(nx)))


def ricker(freq, nt, dt, delay=None):
    """Unit-amplitude Ricker wavelet sampled at t = n dt, n = 0..nt-1."""
    if delay is None:
        delay = 1.5 / freq
    tau = np.arange(nt, dtype=np.float64) * dt - delay
    arg = (math.pi * freq * tau) ** 2
    return (1.0 - 2.0 * arg) * np.exp(-arg)


def spread(n, count):
    """Evenly spread ``count`` positions over ``n`` cells: floor((i+1/2) n/count)."""
    return np.array([int(math.floor((i + 0.5) * n / count)) for i in range(count)], dtype=np.int64)


def pad_model(interior, pml, p):
    """Edge-replicate an interior model into the CPML band and the halo."""
    return np.pad(np.asarray(interior, dtype=np.float64), pml + p, mode="edge")


def layered(rng, n_int, n_layers, eps_lo, eps_hi, sig_lo, sig_hi):
    """Flat layers with seeded distinct sorted interface depths."""
    depths = np.sort(rng.choice(np.arange(1, n_int), size=n_layers - 1, replace=False))
    eps_vals = rng.uniform(eps_lo, eps_hi, size=n_layers)
    sig_vals = rng.uniform(sig_lo, sig_hi, size=n_layers)
    eps = np.empty((n_int, n_int))
    sig = np.empty((n_int, n_int))
    bounds = [0] + list(depths) + [n_int]
    for i in range(n_layers):
        eps[bounds[i]:bounds[i + 1], :] = eps_vals[i]
        sig[bounds[i]:bounds[i + 1], :] = sig_vals[i]
    return eps, sig


def smooth_random(rng, n_int, smooth, lo, hi):
    """Gaussian-filtered N(0,1) noise rescaled to [lo, hi]."""
    from scipy.ndimage import gaussian_filter

    noise = rng.standard_normal((n_int, n_int))
    sm = gaussian_filter(noise, sigma=smooth, mode="reflect")
    sm = (sm - sm.min()) / max(sm.max() - sm.min(), 1e-300)
    return lo + (hi - lo) * sm


def paint_ellipses(rng, eps, sig, count, ax_lo, ax_hi, eps_lo, eps_hi, sig_lo, sig_hi):
    """Paint ``count`` rotated ellipses, in order, onto the interior models."""
    n = eps.shape[0]
    for _ in range(count):
        cy, cx = rng.uniform(0, n, size=2)
        a_ax, b_ax = rng.uniform(ax_lo, ax_hi, size=2)
        th = rng.uniform(0.0, math.pi)
        e_val = rng.uniform(eps_lo, eps_hi)
        s_val = rng.uniform(sig_lo, sig_hi)
        c, s = math.cos(th), math.sin(th)
        # only the bounding box of the ellipse can hold inside points
        rad = max(a_ax, b_ax) + 1.0
        ylo, yhi = max(0, int(cy - rad)), min(n, int(cy + rad) + 1)
        xlo, xhi = max(0, int(cx - rad)), min(n, int(cx + rad) + 1)
        if ylo >= yhi or xlo >= xhi:
            continue
        yy, xx = np.mgrid[ylo:yhi, xlo:xhi].astype(np.float64)
        u = (xx - cx) * c + (yy - cy) * s
        v = -(xx - cx) * s + (yy - cy) * c
        inside = (u / a_ax) ** 2 + (v / b_ax) ** 2 <= 1.0
        eps[ylo:yhi, xlo:xhi][inside] = e_val
        sig[ylo:yhi, xlo:xhi][inside] = s_val
    return eps, sig


# ---------------------------------------------------------------------------
# Assembly
# ---------------------------------------------------------------------------

def assemble(name, order, eps_int, sig_int, npml, h, nt, n_shots, n_rec, freq,
             src_row=2, rec_row=5, dt=None, snap="f32", ckpt_every=0,
             obs_eps_int=None, src_cols=None, mu_int=None, cfl_fraction=0.9, kappa_max=1.0):
    """Build a Workload from an interior model and acquisition parameters."""
    p = order // 2
    ny_int, nx_int = eps_int.shape                  # the interior may be rectangular
    eps_r = pad_model(eps_int, npml, p)
    sigma = pad_model(sig_int, npml, p)
    mu_r = pad_model(np.ones_like(eps_int) if mu_int is None else mu_int, npml, p)
    ny = ny_int + 2 * npml + 2 * p
    nx = nx_int + 2 * npml + 2 * p
    y0 = x0 = p + npml
    y1 = y0 + ny_int
    x1 = x0 + nx_int
    eps_min = float(eps_r.min()) if obs_eps_int is None else float(min(eps_r.min(), obs_eps_int.min()))
    if dt is None:
        dt = stable_dt(eps_min, float(mu_r.min()), h, h, order, cfl_fraction)
    ca, cb, cq = update_coefficients(eps_r, sigma, mu_r, dt)
    vmax = C0 / math.sqrt(eps_min * float(mu_r.min()))
    ycoefs = cpml_axis(ny, y0, y1, npml, h, dt, vmax, freq, kappa_max=kappa_max)
    xcoefs = cpml_axis(nx, x0, x1, npml, h, dt, vmax, freq, kappa_max=kappa_max)
    cpml = pack_cpml(ny, nx, ycoefs, xcoefs)
    wav = ricker(freq, nt, dt)
    f = np.repeat(wav[:, None, None], n_shots, axis=1)          # [nt][S][1]
    if src_cols is None:
        src_cols = spread(nx_int, n_shots)
    src = ((y0 + src_row) * nx + x0 + np.asarray(src_cols, dtype=np.int64))[:, None]
    rec_cols = spread(nx_int, n_rec)
    rec_row_idx = (y0 + rec_row) * nx + x0 + rec_cols
    rec = np.repeat(rec_row_idx[None, :], n_shots, axis=0)
    wl = Workload(
        name=name, order=order, n_shots=n_shots, ny=ny, nx=nx,
        pml_y0=y0, pml_y1=y1, pml_x0=x0, pml_x1=x1, dy=h, dx=h, dt=dt, nt=nt,
        eps_r=eps_r, sigma=sigma, mu_r=mu_r, ca=ca, cb=cb, cq=cq, cpml=cpml,
        f=f, src=src.astype(np.int64), rec=rec.astype(np.int64), freq=freq,
        snap=snap, ckpt_every=ckpt_every,
        obs_eps_r=None if obs_eps_int is None else pad_model(obs_eps_int, npml, p),
    )
    return wl


def observed_coefficients(wl):
    """Ca, Cb, Cq of the observed model of a workload (same dt, sigma, mu_r)."""
    if wl.obs_eps_r is None:
        return None
    return update_coefficients(wl.obs_eps_r, wl.sigma, wl.mu_r, wl.dt)


# ---------------------------------------------------------------------------
# The five workloads (seed = 20260 + config number).  ``n_int``, ``nt`` and
# ``n_shots`` may be overridden to get reduced versions with the same model
# recipe; the model is then generated at the reduced interior size.
# ---------------------------------------------------------------------------

CONFIG_DEFAULTS = {
    1: dict(order=2, n_int=64, npml=10, h=0.02, nt=300, n_shots=1, n_rec=16, freq=500e6, snap="f32", ckpt_every=0),
    2: dict(order=4, n_int=256, npml=20, h=0.01, nt=1000, n_shots=4, n_rec=64, freq=800e6, snap="f32", ckpt_every=0),
    3: dict(order=8, n_int=1024, npml=32, h=0.01, nt=2000, n_shots=16, n_rec=256, freq=600e6, snap="bf16", ckpt_every=0),
    4: dict(order=8, n_int=4096, npml=40, h=0.005, nt=4000, n_shots=8, n_rec=1024, freq=800e6, snap="f32", ckpt_every=64),
    5: dict(order=4, n_int=384, npml=20, h=0.01, nt=800, n_shots=128, n_rec=32, freq=600e6, snap="f32", ckpt_every=0),
}

CONFIG_DESCRIPTIONS = {
    1: "order-2, 64x64 interior + 10-cell CPML, homogeneous eps_r=4, 300 steps, 1 shot, 16 receivers, fp32 snapshots",
    2: "order-4, 256x256 interior + 20-cell CPML, 5 flat layers, 1000 steps, 4 shots, 64 receivers, fp32 snapshots",
    3: "order-8, 1024x1024 interior + 32-cell CPML, smooth random eps_r in [3,15], 2000 steps, 16 shots, 256 receivers, bf16 snapshots",
    4: "order-8, 4096x4096 interior + 40-cell CPML, layers + 30 ellipses, 4000 steps, 8 shots, 1024 receivers, fp32, checkpoint every 64 steps + replay",
    5: "order-4, 384x384 interior + 20-cell CPML, smooth random eps_r in [2,12], 800 steps, 128 shots, 32 receivers, fp32 snapshots",
}


def make_config(cfg: int, **over) -> Workload:
    """Workload ``cfg`` (1..5), optionally reduced via keyword overrides.

    Recognised overrides: n_int, npml, nt, n_shots, n_rec, order, snap,
    ckpt_every, seed, kappa_max (CPML stretching, 1 = none).
    """
    p = dict(CONFIG_DEFAULTS[cfg])
    seed = over.pop("seed", 20260 + cfg)
    kappa_max = over.pop("kappa_max", 1.0)
    p.update(over)
    rng = np.random.default_rng(seed)
    n = p["n_int"]
    obs = None
    src_cols = None
    if cfg == 1:
        eps = np.full((n, n), 4.0)
        sig = np.zeros((n, n))
        yy, xx = np.mgrid[0:n, 0:n].astype(np.float64)
        c = n // 2
        obs = eps + 2.0 * np.exp(-((yy - c) ** 2 + (xx - c) ** 2) / (2.0 * 4.0 ** 2))
    elif cfg == 2:
        eps, sig = layered(rng, n, 5, 1.0, 25.0, 0.0, 0.01)
    elif cfg == 3:
        eps = smooth_random(rng, n, 20.0 * n / 1024.0 if n < 1024 else 20.0, 3.0, 15.0)
        sig = np.full((n, n), 1e-3)
    elif cfg == 4:
        eps, sig = layered(rng, n, 10, 1.0, 30.0, 0.0, 0.05)
        scale = n / 4096.0
        eps, sig = paint_ellipses(rng, eps, sig, 30, 16.0 * scale, 256.0 * scale,
                                  1.0, 30.0, 0.0, 0.05)
    elif cfg == 5:
        eps = smooth_random(rng, n, 10.0 * n / 384.0 if n < 384 else 10.0, 2.0, 12.0)
        sig = np.full((n, n), 0.005)
    else:
        raise ValueError(f"unknown config {cfg}")
    return assemble(
        f"config{cfg}", p["order"], eps, sig, p["npml"], p["h"], p["nt"], p["n_shots"],
        p["n_rec"], p["freq"], snap=p["snap"], ckpt_every=p["ckpt_every"],
        obs_eps_int=obs, src_cols=src_cols, kappa_max=kappa_max,
    )


def random_workload(order, n_int, npml, nt, n_shots, n_src, n_rec, seed, h=0.01,
                    freq=700e6, eps_range=(1.5, 9.0), sig_range=(0.0, 0.02),
                    identity_pml=False, src_anywhere=False, nx_int=None, mu_range=(1.0, 2.0),
                    kappa_max=1.0):
    """A small heterogeneous workload for property tests.

    Models are random per cell (not smooth), several sources per shot at
    random interior cells (duplicates allowed), receivers at random cells,
    and random source amplitudes instead of a wavelet, so that every path
    through the kernels is exercised.  ``mu_range`` = (m, m) gives a
    uniform mu_r = m (non-magnetic media for m = 1); ``kappa_max`` > 1
    stretches the CPML coordinates (kappa from 1 to kappa_max into the band).
    """
    rng = np.random.default_rng(seed)
    shape = (n_int, n_int if nx_int is None else nx_int)   # rows x columns of the interior
    eps = rng.uniform(*eps_range, size=shape)
    sig = rng.uniform(*sig_range, size=shape)
    mu = rng.uniform(*mu_range, size=shape)
    wl = assemble(f"random{seed}", order, eps, sig, npml, h, nt, n_shots, n_rec, freq,
                  mu_int=mu, kappa_max=kappa_max)
    p = order // 2
    lo = p if src_anywhere else wl.pml_y0
    hi_y = (wl.ny - p) if src_anywhere else wl.pml_y1 - 1
    hi_x = (wl.nx - p) if src_anywhere else wl.pml_x1 - 1
    ys = rng.integers(lo, hi_y + 1, size=(n_shots, n_src))
    xs = rng.integers(lo, hi_x + 1, size=(n_shots, n_src))
    wl.src = (ys * wl.nx + xs).astype(np.int64)
    ys = rng.integers(lo, hi_y + 1, size=(n_shots, n_rec))
    xs = rng.integers(lo, hi_x + 1, size=(n_shots, n_rec))
    wl.rec = (ys * wl.nx + xs).astype(np.int64)
    wl.f = rng.standard_normal((nt, n_shots, n_src))
    if identity_pml:
        wl.cpml = identity_cpml(wl.ny, wl.nx)
    return wl


def homogeneous_workload(order, ny, nx, npml, nt, src_yx, rec_yx, seed, eps_r=4.0, h=0.01):
    """One shot in a homogeneous lossless medium with an identity CPML
    profile, sized ny x nx (padded), with one source at ``src_yx`` and
    receivers at the cells ``rec_yx``, random source amplitudes.

    The coefficient arrays are float32 (float32-exact values), so grids
    close to the largest allowed size stay cheap to build; ``eps_r``,
    ``sigma`` and ``mu_r`` are 1x1 placeholders.  Its field after nt steps
    is a translate of the same problem on any grid that keeps the source
    and receivers more than 2 * P * nt cells from the halo.
    """
    rng = np.random.default_rng(seed)
    p = order // 2
    dt = stable_dt(eps_r, 1.0, h, h, order)
    ca, cb, cq = update_coefficients(np.array([eps_r]), np.array([0.0]), np.array([1.0]), dt)
    full = lambda v: np.full((ny, nx), np.float32(v[0]), dtype=np.float32)
    f = rng.standard_normal((nt, 1, 1)).astype(np.float32).astype(np.float64)
    src = np.array([[src_yx[0] * nx + src_yx[1]]], dtype=np.int64)
    rec = np.array([[y * nx + x for (y, x) in rec_yx]], dtype=np.int64)
    one = np.ones((1, 1))
    return Workload(name=f"homogeneous{ny}x{nx}", order=order, n_shots=1, ny=ny, nx=nx,
                    pml_y0=p + npml, pml_y1=ny - p - npml, pml_x0=p + npml, pml_x1=nx - p - npml,
                    dy=h, dx=h, dt=dt, nt=nt, eps_r=one * eps_r, sigma=one * 0.0, mu_r=one,
                    ca=full(ca), cb=full(cb), cq=full(cq), cpml=identity_cpml(ny, nx), f=f, src=src, rec=rec,
                    freq=0.0)


def per_shot_models(wl: Workload, spread: float = 0.25) -> Workload:
    """The same problem with one model per shot (batched models): shot s's
    permittivity is the workload's times 1 + spread * s / (S - 1), which only
    slows the waves, so the workload's dt stays stable.  ``ca``, ``cb``,
    ``cq`` become [S][ny][nx]; ``eps_r`` stays the shared base model."""
    S = wl.n_shots
    coefs = [update_coefficients(wl.eps_r * (1.0 + spread * s / max(S - 1, 1)), wl.sigma, wl.mu_r, wl.dt)
             for s in range(S)]
    ca, cb, cq = (np.stack([c[i] for c in coefs]) for i in range(3))
    return dataclasses.replace(wl, name=wl.name + "-per-shot-models", ca=ca, cb=cb, cq=cq)


def as_f32(wl: Workload) -> Workload:
    """A copy whose float arrays are rounded to float32 and widened back.

    Both the GPU path (which takes float32) and the fp64 oracle then start
    from exactly the same input values.
    """
    out = dataclasses.replace(wl)
    for name in ("ca", "cb", "cq", "cpml", "f"):
        setattr(out, name, getattr(wl, name).astype(np.float32).astype(np.float64))
    return out
