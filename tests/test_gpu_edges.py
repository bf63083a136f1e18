"""GPU parity on edge and degenerate cases, through the C ABI.

Shapes the workload tests do not reach: the smallest grids per order,
rectangular grids (several strips with a ragged last one; a narrow, tall
grid with many chunks), no sources, no receivers, one and two time steps,
checkpoints every step and one step short of nt, and sources and receivers
anywhere in the E set (CPML bands and the set's edge rows and columns
included), several rows per shot.  Every case is compared with the oracle
and, for the two-step forward, bitwise with one step per launch.
"""

import numpy as np
import pytest

from tm_maxwell_fdtd_amd import inputs

from gpu_util import compare, grid_regions, rel_l2, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

REC_TOL = 1e-5
GRAD_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on the CPU)")
    from tm_maxwell_fdtd_amd import native

    native.lib()


def edge_positions(wl, shot, n):
    """n cells on the E set's corners and edges of one shot (y*nx + x)."""
    p = wl.order // 2
    ys = [p, wl.ny - p, p, wl.ny - p, wl.pml_y0, wl.pml_y1 - 1]
    xs = [p, p, wl.nx - p, wl.nx - p, wl.pml_x1 - 1, wl.pml_x0]
    return [ys[(i + shot) % 6] * wl.nx + xs[(i + shot) % 6] for i in range(n)]


CASES = {
    "small-o8": dict(order=8, n_int=1, npml=4, nt=40, n_shots=2, n_src=2, n_rec=3),
    "small-o4": dict(order=4, n_int=1, npml=4, nt=40, n_shots=2, n_src=2, n_rec=3),
    "small-o2": dict(order=2, n_int=2, npml=4, nt=40, n_shots=2, n_src=2, n_rec=3),
    "wide-o8": dict(order=8, n_int=20, npml=6, nx_int=430, nt=50, n_shots=2, n_src=4, n_rec=9),
    "tall-o4": dict(order=4, n_int=330, npml=6, nx_int=18, nt=50, n_shots=2, n_src=4, n_rec=9),
    "no-sources": dict(order=8, n_int=30, npml=6, nt=30, n_shots=2, n_src=0, n_rec=5),
    "no-receivers": dict(order=4, n_int=30, npml=6, nt=30, n_shots=2, n_src=2, n_rec=0),
    "two-steps": dict(order=8, n_int=24, npml=6, nt=2, n_shots=2, n_src=2, n_rec=4),
    "three-steps": dict(order=8, n_int=24, npml=6, nt=3, n_shots=2, n_src=2, n_rec=4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_edge_case(orc, name):
    kw = dict(CASES[name])
    wl = inputs.random_workload(seed=900 + sorted(CASES).index(name), src_anywhere=True, **kw)
    if wl.n_src >= 2:
        wl.src[0, : min(2, wl.n_src)] = edge_positions(wl, 0, min(2, wl.n_src))
    if wl.n_rec >= 2:
        wl.rec[1, : min(3, wl.n_rec)] = edge_positions(wl, 1, min(3, wl.n_rec))
    wl = inputs.as_f32(wl)
    ref = run_oracle(orc, wl)
    got = run_gpu(wl, snap="f32", grad_r=ref["residual"])
    one = run_gpu(wl, snap="f32", grad_r=ref["residual"], time_block=1)
    regions = grid_regions(wl)
    errs = {k: compare(k, got[k], ref[k], tol, regions if k.startswith("gc") else None)
            for k, tol in (("records", REC_TOL), ("gca_shot", GRAD_TOL), ("gcb_shot", GRAD_TOL),
                           ("grad_f", GRAD_TOL))}
    print(f"[{name}] ny {wl.ny} nx {wl.nx} nt {wl.nt}: "
          + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=f"{name} {key}: two-step != one-step")


@pytest.mark.parametrize("order", inputs.ORDERS)
def test_minimal_grid_and_single_step(orc, order):
    """The smallest grids (one CPML cell, one interior cell at orders 4 and 8,
    two at order 2: ny = nx = 2P + 3, resp. 6) and a single time step.  The one-cell CPML damps so hard
    that the interior gradient is rounding noise in both precisions, so the
    gradients are only compared between one and two steps per launch."""
    n_int = 1 if order > 2 else 2
    wl = inputs.random_workload(order, n_int, 1, nt=30, n_shots=2, n_src=2, n_rec=3, seed=960 + order,
                                src_anywhere=True)
    wl.rec[0, 0] = wl.src[0, 0]
    wl = inputs.as_f32(wl)
    ref = run_oracle(orc, wl)
    got = run_gpu(wl, snap="f32", grad_r=ref["residual"])
    one = run_gpu(wl, snap="f32", grad_r=ref["residual"], time_block=1)
    assert rel_l2(got["records"], ref["records"]) <= REC_TOL
    assert rel_l2(got["grad_f"], ref["grad_f"]) <= GRAD_TOL
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=key)
    # a single step: the record of a receiver on a source cell is the source amplitude
    import dataclasses

    w1 = dataclasses.replace(wl, nt=1, f=wl.f[:1].copy())
    r1 = run_gpu(w1, snap="f32")["records"]
    assert r1[0, 0, 0] == np.float32(wl.f[0, 0, 0]) or rel_l2(r1, orc.forward(w1)[0]) <= REC_TOL


@pytest.mark.parametrize("k", [1, 2, 29])
def test_checkpoint_intervals(orc, k):
    """Checkpoints every step, every other step and one step short of nt."""
    wl = inputs.as_f32(inputs.random_workload(8, 30, 6, nt=30, n_shots=2, n_src=2, n_rec=5, seed=950 + k,
                                              src_anywhere=True))
    full = run_gpu(wl, snap="f32", ckpt_every=0)
    ck = run_gpu(wl, snap="f32", ckpt_every=k)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(ck[key], full[key], err_msg=f"K={k} {key}")
    ref = run_oracle(orc, wl)
    assert rel_l2(ck["gca_shot"], ref["gca_shot"]) <= GRAD_TOL


def _run_windowed(wl, grad_r, centre, half):
    """Records, and the per-shot gradients on the window centre +- half
    together with their nonzero counts over the whole grid (so nothing is
    copied back at full size)."""
    import torch

    from tm_maxwell_fdtd_amd import native

    prop = native.Propagator(wl)
    try:
        r = prop.forward(store=True)
        resid = torch.as_tensor(np.asarray(grad_r, np.float32), device=prop.device)
        grad_f, gca, gcb = prop.adjoint(resid)
        win = (slice(centre[0] - half, centre[0] + half + 1), slice(centre[1] - half, centre[1] + half + 1))
        out = dict(records=r.cpu().numpy(), grad_f=grad_f.cpu().numpy(),
                   gca=gca[0][win].cpu().numpy(), gcb=gcb[0][win].cpu().numpy(),
                   nnz_a=int(torch.count_nonzero(gca[0])), nnz_b=int(torch.count_nonzero(gcb[0])))
        torch.cuda.synchronize()
    finally:
        prop.close()
    return out


def test_largest_grid_matches_a_small_one(orc):
    """The largest square grid one buffer view allows (order 4), with the
    source 40 cells from its far corner: in a homogeneous lossless medium
    the records and gradients of 6 steps equal bitwise those of the same
    source and receivers on an 80 x 80 grid (the fields reach at most 24
    cells), which match the oracle; the gradients are zero outside the
    window.  This runs every offset and buffer view at its largest."""
    from gpu_util import largest_square_grid

    order, npml, nt, half = 4, 8, 6, 30
    n = largest_square_grid(order, npml)
    offs = [(0, 4), (-3, 0), (5, -2), (2, 7), (-6, -6)]
    big_c, small_c = (n - 40, n - 40), (40, 40)
    big = inputs.homogeneous_workload(order, n, n, npml, nt, big_c, [(big_c[0] + a, big_c[1] + b) for a, b in offs],
                                      seed=910)
    small = inputs.homogeneous_workload(order, 80, 80, npml, nt, small_c,
                                        [(small_c[0] + a, small_c[1] + b) for a, b in offs], seed=910)
    print(f"[largest grid] {n} x {n}", flush=True)
    ref = run_oracle(orc, small)
    got_s = _run_windowed(small, ref["residual"], small_c, half)
    got_b = _run_windowed(big, ref["residual"], big_c, half)
    e_r = rel_l2(got_b["records"], ref["records"])
    e_a = rel_l2(got_b["gca"], ref["gca_shot"][0][10:71, 10:71])
    e_b = rel_l2(got_b["gcb"], ref["gcb_shot"][0][10:71, 10:71])
    print(f"[largest grid] records {e_r:.2e}  gCa {e_a:.2e}  gCb {e_b:.2e}", flush=True)
    assert e_r <= REC_TOL and e_a <= GRAD_TOL and e_b <= GRAD_TOL
    for key in ("records", "grad_f", "gca", "gcb"):
        np.testing.assert_array_equal(got_b[key], got_s[key], err_msg=key)
    assert got_b["nnz_a"] == np.count_nonzero(got_b["gca"]) > 0
    assert got_b["nnz_b"] == np.count_nonzero(got_b["gcb"]) > 0
