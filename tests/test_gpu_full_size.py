"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (all shots, full grid, full time range, the workload's
snapshot type and checkpoint mode), and over the full time length of the
long workloads on reduced grids.

The oracle cannot run every full-size problem, so the checks are sampled:
  * shots are independent, so selected shots of the full batch are compared
    with oracle runs of those shots alone;
  * the first T records do not depend on later steps, and an adjoint whose
    residual vanishes after step T only involves steps before T, so records
    and gradients of a time window are compared with a T-step oracle run
    (config 4's gradients only; its records are compared over all 4000
    steps, and the same recipe runs all 4000 steps with gradients on a
    reduced grid);
  * the shot sum is checked against the fp64 sum of the GPU's own per-shot
    gradients, and the adjoint against the forward with a dot test (both hold
    at any size).
Long oracle runs use its segment-replay adjoint (bitwise the full-storage
one) and print a progress line per segment.  Every array is compared by
relative L2, element by element and region by region (``compare``).
"""

import numpy as np
import pytest

from tm_maxwell_fdtd_amd import inputs

from gpu_util import compare, grid_regions, rel_l2, run_gpu, run_gpu_window, sub_workload

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


@pytest.fixture
def say(capsys):
    """Print a progress line past pytest's capture (long oracle runs)."""
    def _say(msg):
        with capsys.disabled():
            print(f"    [{msg}]", flush=True)
    return _say


def check_shots(wl, got, ref, shots, tw, label, grads=True):
    """GPU outputs of ``shots`` (first ``tw`` steps) against oracle outputs
    of those shots alone."""
    tol = GRAD_TOL[wl.snap]
    regions = grid_regions(wl)
    e = {"records": compare("records", got["records"][:tw, shots], ref["records"], REC_TOL)}
    if grads:
        e["gCa"] = compare("gCa/shot", got["gca_shot"][shots], ref["gca_shot"], tol, regions)
        e["gCb"] = compare("gCb/shot", got["gcb_shot"][shots], ref["gcb_shot"], tol, regions)
        e["grad_f"] = compare("grad_f", got["grad_f"][:tw, shots], ref["grad_f"], max(tol, 1e-4))
        # shot sum against the fp64 sum of the GPU's per-shot gradients
        e["shot-sum"] = max(rel_l2(got["gca"], got["gca_shot"].astype(np.float64).sum(axis=0)),
                            rel_l2(got["gcb"], got["gcb_shot"].astype(np.float64).sum(axis=0)))
    print(f"[{label}] shots {shots} steps<{tw}: " + "  ".join(f"{k} {v:.2e}" for k, v in e.items()), flush=True)
    if grads:
        assert e["shot-sum"] <= SUM_TOL, e
        # masked cells are exactly zero
        mask = np.zeros((wl.ny, wl.nx), bool)
        mask[wl.pml_y0:wl.pml_y1, wl.pml_x0:wl.pml_x1] = True
        assert not np.any(got["gca_shot"][:, ~mask]) and not np.any(got["gcb_shot"][:, ~mask])
    return e


def compare_sampled(orc, wl, got, shots, t_window, label):
    """Records and per-shot gradients of the sampled shots against
    full-storage oracle runs of those shots alone over the first
    ``t_window`` steps (all when None)."""
    tw = wl.nt if t_window is None else t_window
    sub = sub_workload(wl, shots, tw)
    r_o, _, snaps = orc.forward(sub, store=True)
    # the adjoint of the same float32 residual the GPU used
    resid = got["residual"][:tw, shots].astype(np.float64)
    assert np.all(got["residual"][tw:] == 0)
    gf_o, gca_o, gcb_o = orc.adjoint(sub, resid, snaps)
    del snaps
    # the adjoint state is exactly zero after the window
    assert np.all(got["grad_f"][tw:] == 0)
    ref = dict(records=r_o, gca_shot=gca_o, gcb_shot=gcb_o, grad_f=gf_o)
    return check_shots(wl, got, ref, shots, tw, label)


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
def test_config3_full_all_steps(orc, say):
    """Order 8, 1096^2, 16 shots, 2000 steps, bf16 snapshots: shots 0 and 15,
    records and the gradients of J = 1/2 |r|^2 over all 2000 steps (the
    oracle replays 100-step segments from checkpoints, fp64 snapshots)."""
    wl = inputs.as_f32(inputs.make_config(3))
    got = run_gpu_window(wl)
    shots = [0, 15]
    sub = sub_workload(wl, shots)
    resid = got["residual"][:, shots].astype(np.float64)
    ref = orc.gradient_checkpointed(sub, 100, grad_r=resid, progress=say)
    check_shots(wl, got, ref, shots, wl.nt, "config3 full, all steps")


@pytest.fixture(scope="module")
def config4_run():
    """Order 8, 4184^2, 8 shots, 4000 steps, checkpoints every 64 steps with
    segment replay: the full forward (all records), and the adjoint of the
    residual of the first 70 steps (two replayed segments)."""
    wl = inputs.as_f32(inputs.make_config(4))
    assert wl.ckpt_every == 64
    return wl, run_gpu_window(wl, t_window=70)


@pytest.mark.timeout(900)
def test_config4_full_window_gradients(orc, config4_run):
    """Gradients, grad_f and records of shots 0 and 7 over the first 70
    steps (the fp64 oracle at this grid size keeps about 0.27 GB of
    snapshots per step and shot)."""
    wl, got = config4_run
    compare_sampled(orc, wl, got, [0, 7], 70, "config4 full")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("shot", [0, 7])
def test_config4_full_records_all_steps(orc, config4_run, say, shot):
    """Records of one shot over all 4000 steps against an oracle forward of
    that shot alone (about 7e10 cell-updates in fp64, run in 250-step
    chunks)."""
    wl, got = config4_run
    sub = sub_workload(wl, [shot])
    st = None
    r = np.zeros((wl.nt, 1, wl.n_rec))
    for t0 in range(0, wl.nt, 250):
        t1 = min(t0 + 250, wl.nt)
        _, st, _ = orc.forward(sub, t0, t1, state=st, records=r)
        say(f"config4 shot {shot}: oracle forward {t1}/{wl.nt}")
    check_shots(wl, got, dict(records=r), [shot], wl.nt, f"config4 full records shot {shot}", grads=False)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,over,every", [
    (4, dict(n_int=256, n_shots=2, n_rec=64), 64),      # 4000 steps, 62 replayed segments
    (3, dict(n_int=256, n_shots=2, n_rec=64), 100),     # 2000 steps, bf16 snapshots
])
def test_full_length_reduced_grid(orc, say, cfg, over, every):
    """The long workloads' recipes over their full time length (config 4:
    4000 steps with checkpoints every 64 steps and segment replay on the
    GPU; config 3: 2000 steps with bf16 snapshots) on a 256^2 interior:
    records, per-shot gradients and grad_f of J = 1/2 |r|^2 over every step
    against the oracle (fp32 drift over the whole run, every replay)."""
    wl = inputs.as_f32(inputs.make_config(cfg, **over))
    got = run_gpu(wl)
    ref = orc.gradient_checkpointed(wl, every, grad_r=got["residual"].astype(np.float64), progress=say)
    check_shots(wl, got, ref, list(range(wl.n_shots)), wl.nt, f"config{cfg} recipe, 256^2, all {wl.nt} steps")


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
