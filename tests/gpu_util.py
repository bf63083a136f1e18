"""Helpers shared by the GPU tests: run a workload through the C ABI and
through the oracle, and compare."""

from __future__ import annotations

import numpy as np

from tm_maxwell_fdtd_amd import inputs


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def seam_columns(wl, halo=None):
    """Columns within ``halo`` cells of a strip edge of the step kernels:
    one-step strips are 256 - 4P + 2 columns wide; the two-step kernels
    cut the columns into as many strips of at most 256 - 8P + 4 as needed,
    of equal widths; both start at column P."""
    p = wl.order // 2
    halo = 4 * p if halo is None else halo
    nx_e = wl.nx - 2 * p + 1
    w0 = 256 - 8 * p + 4
    n2 = -(-nx_e // w0)
    cols = set()
    for w in (256 - 4 * p + 2, -(-nx_e // n2)):
        for c0 in range(p, wl.nx, w):
            cols.update(range(max(0, c0 - halo), min(wl.nx, c0 + halo)))
    return np.array(sorted(cols), dtype=np.int64)


def grid_regions(wl):
    """Boolean [ny][nx] masks of the places where a localized kernel error
    would hide in a global norm: the interior rows and columns next to the
    CPML bands (2P deep) and the strip seams inside the interior window."""
    p = wl.order // 2
    y0, y1, x0, x1 = wl.pml_y0, wl.pml_y1, wl.pml_x0, wl.pml_x1
    inside = np.zeros((wl.ny, wl.nx), bool)
    inside[y0:y1, x0:x1] = True
    regions = {}
    m = np.zeros_like(inside)
    m[y0:y0 + 2 * p] = True
    m[y1 - 2 * p:y1] = True
    regions["band rows"] = m & inside
    m = np.zeros_like(inside)
    m[:, x0:x0 + 2 * p] = True
    m[:, x1 - 2 * p:x1] = True
    regions["band cols"] = m & inside
    m = np.zeros_like(inside)
    m[:, seam_columns(wl)] = True
    regions["strip seams"] = m & inside
    return regions


def compare(name, got, ref, tol, regions=None, elem_factor=10.0):
    """Relative L2 of ``got`` against ``ref``, plus two local bounds:
    every element within elem_factor * tol * max|ref|, and the relative L2
    of each region (masks over the last two axes) within tol.  Returns the
    global relative L2; raises AssertionError naming the failing bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    e = rel_l2(got, ref)
    assert e <= tol, f"{name}: relative L2 {e:.3e} > {tol:.1e}"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if ref.size:
        worst = float(np.abs(got - ref).max())
        assert worst <= elem_factor * tol * scale + 1e-30, \
            f"{name}: max element error {worst:.3e} > {elem_factor:g} x {tol:.1e} x max|ref| ({scale:.3e})"
    for rname, mask in (regions or {}).items():
        if not mask.any():
            continue
        g, r = got[..., mask], ref[..., mask]
        nr = np.linalg.norm(r)
        if nr == 0.0:
            assert not np.any(g), f"{name} [{rname}]: nonzero where the reference is 0"
            continue
        er = float(np.linalg.norm(g - r) / nr)
        assert er <= tol, f"{name} [{rname}]: relative L2 {er:.3e} > {tol:.1e}"
    return e


def observed_records_oracle(orc, wl):
    """Observed data of a workload with an anomaly model (oracle side)."""
    obs = inputs.observed_coefficients(wl)
    if obs is None:
        return None
    ca, cb, cq = (np.asarray(x, np.float32).astype(np.float64) for x in obs)
    r, _, _ = orc.forward(wl, ca=ca, cb=cb, cq=cq)
    return r


def run_oracle(orc, wl, observed=None):
    return orc.misfit_and_gradient(wl, observed=observed)


def run_gpu(wl, observed=None, snap=None, ckpt_every=None, grad_r=None, obs_coefs=None, time_block=0,
            storage=0, step_ratio=0, chunks=None):
    """Forward (storing), residual, adjoint and shot sum on the GPU.

    ``storage`` / ``step_ratio`` / ``time_block`` are the plan options of the
    same names; ``chunks`` runs the forward in time chunks split at those steps.

    ``observed``: records of the observed model, a numpy array, or the
    string "gpu" to compute them on the GPU from the workload's observed
    model.  Returns numpy arrays.
    """
    import torch

    from tm_maxwell_fdtd_amd import native

    prop = native.Propagator(wl, snap=snap, ckpt_every=ckpt_every, time_block=time_block, storage=storage,
                             step_ratio=step_ratio)
    try:
        if chunks is None:
            r = prop.forward(store=True)
        else:                                   # the forward in time chunks [0, c1), [c1, c2), ...
            r = None
            bounds = [0, *chunks, wl.nt]
            for t0, t1 in zip(bounds, bounds[1:]):
                r = prop.forward(r=r, store=True, t0=t0, t1=t1)
        if grad_r is not None:
            resid = torch.as_tensor(np.asarray(grad_r, np.float32), device=prop.device)
        elif observed is None:
            resid = r
        else:
            d = torch.as_tensor(np.asarray(observed, np.float32), device=prop.device)
            resid = (r - d).contiguous()
        grad_f, gca, gcb = prop.adjoint(resid)
        ga, gb = prop.grad(gca, gcb)
        torch.cuda.synchronize()
        out = dict(records=r.cpu().numpy(), grad_f=grad_f.cpu().numpy(), gca_shot=gca.cpu().numpy(),
                   gcb_shot=gcb.cpu().numpy(), gca=ga.cpu().numpy(), gcb=gb.cpu().numpy(),
                   residual=resid.cpu().numpy())
    finally:
        prop.close()
    return out


def gpu_observed(wl):
    """Records of the workload's observed model computed on the GPU."""
    import dataclasses

    import torch

    from tm_maxwell_fdtd_amd import native

    ca, cb, cq = inputs.observed_coefficients(wl)
    w2 = dataclasses.replace(wl, ca=ca, cb=cb, cq=cq)
    prop = native.Propagator(w2)
    try:
        r = prop.forward(store=False)
        torch.cuda.synchronize()
        return r.cpu().numpy()
    finally:
        prop.close()


def sub_workload(wl, shots, nt=None):
    """The same problem restricted to some shots and the first ``nt`` steps.

    Shots are independent and the first nt records of a run do not depend on
    later steps, so the oracle can check sampled outputs of a full-size run.
    """
    import dataclasses

    shots = list(shots)
    nt = wl.nt if nt is None else nt
    return dataclasses.replace(wl, n_shots=len(shots), nt=nt, f=wl.f[:nt, shots].copy(),
                               src=wl.src[shots].copy(), rec=wl.rec[shots].copy())


def run_gpu_window(wl, t_window=None):
    """Full-size GPU run: forward with storage, then the adjoint of
    J = 1/2 |r|^2 restricted to time steps t < t_window (grad_r = r there,
    0 later; None = all steps), the shot sum, and the residual used."""
    import torch

    from tm_maxwell_fdtd_amd import native

    prop = native.Propagator(wl)
    try:
        r = prop.forward(store=True)
        resid = r.clone()
        if t_window is not None:
            resid[t_window:] = 0
        grad_f, gca, gcb = prop.adjoint(resid)
        ga, gb = prop.grad(gca, gcb)
        torch.cuda.synchronize()
        out = dict(records=r.cpu().numpy(), grad_f=grad_f.cpu().numpy(), gca_shot=gca.cpu().numpy(),
                   gcb_shot=gcb.cpu().numpy(), gca=ga.cpu().numpy(), gcb=gb.cpu().numpy(),
                   residual=resid.cpu().numpy())
        del r, resid, grad_f, gca, gcb, ga, gb
    finally:
        prop.close()
        del prop
        torch.cuda.empty_cache()
    return out


def shot_block_bytes(n, npml, order):
    """Bytes of one shot's state block on an n x n padded grid: Ey, Hx, Hz
    and the y- and x-band memories of both updates, each 256-byte aligned."""
    al = lambda v: (v + 255) // 256 * 256
    p = order // 2
    band = (p + npml) + (n - (n - p - npml) + 1)      # rows below y0 and from y1-1 on
    return 3 * al(n * n * 4) + 2 * al(band * n * 4) + 2 * al(n * band * 4)


def largest_square_grid(order, npml):
    """The largest n whose shot block fits one buffer view (2^31 - 256 bytes)."""
    n = 1024
    while shot_block_bytes(n + 1, npml, order) <= (1 << 31) - 256:
        n += 1
    return n
