"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (all shots, full grid, full time range, the workload's
snapshot type and checkpoint mode).

The oracle cannot run every full-size problem, so the checks are sampled:
  * shots are independent, so selected shots of the full batch are compared
    with oracle runs of those shots alone;
  * the first T records do not depend on later steps, and an adjoint whose
    residual vanishes after step T only involves steps before T, so records
    and gradients of a time window are compared with a T-step oracle run;
  * the shot sum is checked against the fp64 sum of the GPU's own per-shot
    gradients, and the adjoint against the forward with a dot test (both hold
    at any size).
Tolerances are those of the reduced parity tests.
"""

import numpy as np
import pytest

from tm_maxwell_fdtd_amd import inputs

from gpu_util import rel_l2, run_gpu_window, sub_workload

pytestmark = pytest.mark.gpu

REC_TOL = 1e-5
GRAD_TOL = {"f32": 1e-4, "bf16": 2e-2}
SUM_TOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on the CPU)")
    from tm_maxwell_fdtd_amd import native

    native.lib()


def compare_sampled(orc, wl, got, shots, t_window, label):
    """Records (all steps, or the window) and per-shot gradients of the
    sampled shots against oracle runs of those shots alone."""
    tw = wl.nt if t_window is None else t_window
    tol = GRAD_TOL[wl.snap]
    # records over the window (all steps when t_window is None)
    sub = sub_workload(wl, shots, tw)
    r_o, _, snaps = orc.forward(sub, store=True)
    e_r = rel_l2(got["records"][:tw, shots], r_o)
    # the adjoint of the same float32 residual the GPU used
    resid = got["residual"][:tw, shots].astype(np.float64)
    assert np.all(got["residual"][tw:] == 0)
    gf_o, gca_o, gcb_o = orc.adjoint(sub, resid, snaps)
    del snaps
    e_a = rel_l2(got["gca_shot"][shots], gca_o)
    e_b = rel_l2(got["gcb_shot"][shots], gcb_o)
    e_f = rel_l2(got["grad_f"][:tw, shots], gf_o)
    # the adjoint state is exactly zero after the window
    assert np.all(got["grad_f"][tw:] == 0)
    # shot sum against the fp64 sum of the GPU's per-shot gradients
    e_sa = rel_l2(got["gca"], got["gca_shot"].astype(np.float64).sum(axis=0))
    e_sb = rel_l2(got["gcb"], got["gcb_shot"].astype(np.float64).sum(axis=0))
    print(f"[{label}] shots {shots} steps<{tw}: records {e_r:.2e}  gCa {e_a:.2e}  gCb {e_b:.2e}  "
          f"grad_f {e_f:.2e}  shot-sum {max(e_sa, e_sb):.2e}", flush=True)
    assert e_r <= REC_TOL, e_r
    assert e_a <= tol and e_b <= tol, (e_a, e_b)
    assert e_f <= max(tol, 1e-4), e_f
    assert e_sa <= SUM_TOL and e_sb <= SUM_TOL, (e_sa, e_sb)
    # masked cells are exactly zero
    mask = np.zeros((wl.ny, wl.nx), bool)
    mask[wl.pml_y0:wl.pml_y1, wl.pml_x0:wl.pml_x1] = True
    assert not np.any(got["gca_shot"][:, ~mask]) and not np.any(got["gcb_shot"][:, ~mask])


@pytest.mark.timeout(900)
def test_config2_full(orc):
    """Order 4, 300^2, 4 shots, 1000 steps, fp32 snapshots: every shot, every step."""
    wl = inputs.as_f32(inputs.make_config(2))
    got = run_gpu_window(wl)
    compare_sampled(orc, wl, got, [0, 1, 2, 3], None, "config2 full")


@pytest.mark.timeout(900)
def test_config5_full_sampled_shots(orc):
    """Order 4, 428^2, 128 shots, 800 steps, fp32 snapshots: shots 0 and 127."""
    wl = inputs.as_f32(inputs.make_config(5))
    got = run_gpu_window(wl)
    compare_sampled(orc, wl, got, [0, 127], None, "config5 full")


@pytest.mark.timeout(900)
def test_config3_full_sampled(orc):
    """Order 8, 1096^2, 16 shots, 2000 steps, bf16 snapshots: shots 0 and 15,
    records over all 2000 steps, gradients of the residual of the first 200."""
    wl = inputs.as_f32(inputs.make_config(3))
    got = run_gpu_window(wl, t_window=200)
    shots = [0, 15]
    r_full, _, _ = orc.forward(sub_workload(wl, shots))
    e_full = rel_l2(got["records"][:, shots], r_full)
    print(f"[config3 full] records over all {wl.nt} steps: {e_full:.2e}", flush=True)
    assert e_full <= REC_TOL, e_full
    compare_sampled(orc, wl, got, shots, 200, "config3 full")


@pytest.mark.timeout(900)
def test_config4_full_sampled(orc):
    """Order 8, 4184^2, 8 shots, 4000 steps, checkpoints every 64 steps with
    segment replay: shots 0 and 7 over the first 70 steps, so the gradient
    takes snapshots from two replayed segments (the fp64 oracle at this grid
    size keeps about 0.27 GB of snapshots per step and shot)."""
    wl = inputs.as_f32(inputs.make_config(4))
    assert wl.ckpt_every == 64
    got = run_gpu_window(wl, t_window=70)
    compare_sampled(orc, wl, got, [0, 7], 70, "config4 full")


@pytest.mark.timeout(900)
def test_config3_full_dot_test():
    """<F f, d> = <f, F^T d> for the wavelet-to-records map at full size."""
    import torch

    from tm_maxwell_fdtd_amd import native

    wl = inputs.as_f32(inputs.make_config(3))
    prop = native.Propagator(wl)
    try:
        r = prop.forward(store=False)
        d = torch.randn(r.shape, generator=torch.Generator().manual_seed(3)).to(prop.device)
        grad_f, _, _ = prop.adjoint(d, want_grads=False)
        lhs = float((r.double() * d.double()).sum())
        rhs = float((prop.f.double() * grad_f.double()).sum())
    finally:
        prop.close()
        del prop
        torch.cuda.empty_cache()
    print(f"[config3 full dot] <Ff,d> {lhs:.9e}  <f,F^T d> {rhs:.9e}  rel {abs(lhs - rhs) / abs(lhs):.2e}",
          flush=True)
    assert abs(lhs - rhs) <= 1e-4 * abs(lhs), (lhs, rhs)
