"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: records relative L2 <= 1e-5; gradients dJ/dCa, dJ/dCb (and the
source gradient) relative L2 <= 1e-4 with float32 snapshots and <= 2e-2
with bfloat16 snapshots.  Both sides start from the same float32 inputs
(``inputs.as_f32``).  Sizes are reduced versions of the five workloads
(same recipes) that span several 64x4 tiles with ragged tails.
"""

import numpy as np
import pytest

from tm_maxwell_fdtd_amd import inputs

from gpu_util import compare, gpu_observed, grid_regions, observed_records_oracle, rel_l2, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

REC_TOL = 1e-5
GRAD_TOL = {"f32": 1e-4, "bf16": 2e-2}
# FP8 snapshots against the oracle's FP8-quantized snapshots: both sides
# quantize float32 values, whose fp32/fp64 differences (~1e-7) flip a code
# only for values within that distance of a rounding midpoint.
FP8_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on the CPU)")
    from tm_maxwell_fdtd_amd import native

    native.lib()


def check(orc, wl, observed_orc=None, snap=None, ckpt_every=None, label="", time_block=0):
    """Records, gradients and grad_f of the GPU path against the oracle.

    tm_adjoint takes dJ/dr as an input; both sides get the same residual
    (the oracle's, rounded to float32 for the GPU), so the comparison
    measures the propagator and not the conditioning of a misfit.  Each
    array is checked by its relative L2 error, element by element (within
    10 x tol x max|ref|) and, for the gradients, region by region (interior
    rows and columns next to the CPML bands, strip seams; ``compare``).
    """
    snap = wl.snap if snap is None else snap
    ref = run_oracle(orc, wl, observed=observed_orc)
    got = run_gpu(wl, snap=snap, ckpt_every=ckpt_every, grad_r=ref["residual"], time_block=time_block)
    tol = GRAD_TOL[snap]
    regions = grid_regions(wl)
    e_r = compare("records", got["records"], ref["records"], REC_TOL)
    e_a = compare("gCa", got["gca"], ref["gca"], tol, regions)
    e_b = compare("gCb", got["gcb"], ref["gcb"], tol, regions)
    e_f = compare("grad_f", got["grad_f"], ref["grad_f"], max(tol, 1e-4))
    e_as = compare("gCa/shot", got["gca_shot"], ref["gca_shot"], tol, regions)
    e_bs = compare("gCb/shot", got["gcb_shot"], ref["gcb_shot"], tol, regions)
    print(f"[{label}] records {e_r:.2e}  gCa {e_a:.2e}  gCb {e_b:.2e}  grad_f {e_f:.2e}  "
          f"per shot {max(e_as, e_bs):.2e}", flush=True)
    # masked cells are exactly zero
    mask = np.zeros((wl.ny, wl.nx), bool)
    mask[wl.pml_y0:wl.pml_y1, wl.pml_x0:wl.pml_x1] = True
    assert np.all(got["gca_shot"][:, ~mask] == 0) and np.all(got["gcb_shot"][:, ~mask] == 0)
    return got, ref


def test_config1_full_size(orc):
    wl = inputs.as_f32(inputs.make_config(1))
    d_orc = observed_records_oracle(orc, wl)
    d_gpu = gpu_observed(wl)
    assert rel_l2(d_gpu, d_orc) <= REC_TOL
    _, ref = check(orc, wl, observed_orc=d_orc, label="config1")
    # End to end, with the residual r - d formed from the GPU's own records of
    # both models.  The subtraction cancels most of the records, so the
    # residual's error is the records' error times |r| / |r - d|.  The adjoint
    # is then checked against the oracle's adjoint of that same float32
    # residual (the map from residual to gradients is linear and fixed by the
    # forward snapshots), so no conditioning enters the gradient comparison.
    e2e = run_gpu(wl, observed=d_gpu, snap="f32")
    e_res = rel_l2(e2e["residual"], ref["residual"])
    cond = np.linalg.norm(ref["records"]) / np.linalg.norm(ref["residual"])
    _, _, snaps = orc.forward(wl, store=True)
    gf2, gca2, gcb2 = orc.adjoint(wl, e2e["residual"].astype(np.float64), snaps)
    errs = dict(gca=rel_l2(e2e["gca"], orc.shot_sum(gca2)), gcb=rel_l2(e2e["gcb"], orc.shot_sum(gcb2)),
                grad_f=rel_l2(e2e["grad_f"], gf2))
    print(f"[config1 end-to-end] residual {e_res:.2e} (|r|/|r-d| = {cond:.0f})  "
          + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    assert e_res <= 2 * REC_TOL * cond
    for key, v in errs.items():
        assert v <= GRAD_TOL["f32"], key


@pytest.mark.parametrize("cfg,over", [
    (2, dict(n_int=100, nt=300, n_shots=4, n_rec=20)),
    (3, dict(n_int=120, nt=300, n_shots=3, n_rec=24)),
    (4, dict(n_int=100, nt=200, n_shots=2, n_rec=32, ckpt_every=64)),
    (5, dict(n_int=96, nt=250, n_shots=8, n_rec=12)),
])
def test_reduced_configs(orc, cfg, over):
    wl = inputs.as_f32(inputs.make_config(cfg, **over))
    check(orc, wl, label=f"config{cfg}-reduced")


@pytest.mark.parametrize("order", inputs.ORDERS)
def test_random_heterogeneous(orc, order):
    wl = inputs.as_f32(inputs.random_workload(order, 70, 9, nt=160, n_shots=3, n_src=3, n_rec=7,
                                              seed=100 + order, src_anywhere=True))
    # duplicate and negative indices
    wl.src[1, 1] = wl.src[1, 0]
    wl.src[2, 2] = -1
    wl.rec[0, 3] = wl.rec[0, 2]
    wl.rec[2, 0] = -1
    wl.rec[1, 4] = wl.src[1, 0]          # receiver on a source cell
    check(orc, wl, snap="f32", label=f"random-o{order}")


@pytest.mark.parametrize("order", inputs.ORDERS)
def test_bf16_snapshots(orc, order):
    wl = inputs.as_f32(inputs.random_workload(order, 60, 8, nt=140, n_shots=2, n_src=1, n_rec=9,
                                              seed=200 + order))
    check(orc, wl, snap="bf16", label=f"bf16-o{order}")


@pytest.mark.parametrize("order", inputs.ORDERS)
def test_gpu_dot_test(order):
    import torch

    from tm_maxwell_fdtd_amd import native

    wl = inputs.as_f32(inputs.random_workload(order, 50, 8, nt=120, n_shots=2, n_src=3, n_rec=6,
                                              seed=300 + order, src_anywhere=True))
    prop = native.Propagator(wl)
    try:
        r = prop.forward(store=False)
        d = torch.randn(r.shape, generator=torch.Generator().manual_seed(order)).to(prop.device)
        grad_f, _, _ = prop.adjoint(d, want_grads=False)
        lhs = float((r.double() * d.double()).sum())
        rhs = float((prop.f.double() * grad_f.double()).sum())
    finally:
        prop.close()
    assert abs(lhs - rhs) <= 1e-5 * abs(lhs), (lhs, rhs)


def test_deterministic_and_chunked():
    import torch

    from tm_maxwell_fdtd_amd import native

    wl = inputs.as_f32(inputs.random_workload(8, 80, 10, nt=90, n_shots=3, n_src=2, n_rec=8, seed=401))
    prop = native.Propagator(wl)
    try:
        r1 = prop.forward(store=True)
        _, a1, b1 = prop.adjoint(r1)
        r2 = torch.zeros_like(r1)
        prop.forward(r=r2, store=True, t0=0, t1=37)
        prop.forward(r=r2, store=True, t0=37, t1=90)
        _, a2, b2 = prop.adjoint(r2)
        torch.cuda.synchronize()
        assert torch.equal(r1, r2)
        assert torch.equal(a1, a2) and torch.equal(b1, b2)
    finally:
        prop.close()


@pytest.mark.parametrize("order,n_int,nx_int,npml,shots", [
    (8, 40, 200, 240, 2),      # x bands wider than a strip: two band strips on the left
    (4, 60, 500, 130, 3),      # two band strips on the right, one on the left
    (2, 50, 1000, 12, 1),      # three interior strips
])
def test_balanced_tiling_bitwise(monkeypatch, order, n_int, nx_int, npml, shots):
    """The cost-balanced cut of the two-step kernels' strips into chunks
    (more, shorter chunks for band strips, chunk edges at weighted row
    quantiles; forced on these small grids with TM_FDTD_BALANCE=2) gives
    bitwise the records, per-shot gradients and grad_f of the uniform cut."""
    wl = inputs.as_f32(inputs.random_workload(order, n_int, npml, nt=40, n_shots=shots, n_src=2, n_rec=6,
                                              seed=611 + order, nx_int=nx_int))
    wl.rec = np.concatenate([wl.src, wl.src + 1, wl.src + wl.nx], axis=1)   # receivers by the sources
    monkeypatch.setenv("TM_FDTD_BALANCE", "0")
    uni = run_gpu(wl, snap="f32", time_block=2)
    monkeypatch.setenv("TM_FDTD_BALANCE", "2")
    bal = run_gpu(wl, snap="f32", time_block=2)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(bal[key], uni[key], err_msg=f"order {order} {key}")
    assert np.abs(uni["records"]).max() > 0


def test_checkpoint_replay_bitwise_equals_full_store():
    wl = inputs.as_f32(inputs.random_workload(4, 64, 8, nt=150, n_shots=2, n_src=1, n_rec=6, seed=501))
    full = run_gpu(wl, snap="f32", ckpt_every=0)
    for k in (16, 64, 149):
        ck = run_gpu(wl, snap="f32", ckpt_every=k)
        for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
            np.testing.assert_array_equal(ck[key], full[key], err_msg=f"K={k} {key}")


def test_batched_shots_bitwise_equal_single_shots():
    import dataclasses

    wl = inputs.as_f32(inputs.random_workload(8, 60, 8, nt=80, n_shots=3, n_src=2, n_rec=5, seed=601))
    allr = run_gpu(wl, snap="f32")
    for s in range(3):
        one = dataclasses.replace(wl, n_shots=1, src=wl.src[s:s + 1].copy(), rec=wl.rec[s:s + 1].copy(),
                                  f=wl.f[:, s:s + 1].copy())
        o = run_gpu(one, snap="f32")
        np.testing.assert_array_equal(o["records"][:, 0], allr["records"][:, s])
        np.testing.assert_array_equal(o["gca_shot"][0], allr["gca_shot"][s])
        np.testing.assert_array_equal(o["gcb_shot"][0], allr["gcb_shot"][s])


@pytest.mark.parametrize("order", inputs.ORDERS)
@pytest.mark.parametrize("snap,ckpt", [("f32", 0), ("bf16", 0), ("fp8", 0), ("f32", 7)])
def test_two_step_launch_bitwise_equals_single_steps(order, snap, ckpt):
    """Two time steps per launch (with the first step's sources and receivers
    inside the kernel) give bitwise the state, records and gradients of one
    step per launch; odd nt and an odd checkpoint interval split pairs."""
    wl = inputs.as_f32(inputs.random_workload(order, 70, 9, nt=101, n_shots=3, n_src=3, n_rec=7,
                                              seed=700 + order, src_anywhere=True))
    wl.src[1, 1] = wl.src[1, 0]          # duplicate source cell
    wl.src[2, 2] = -1
    wl.rec[0, 3] = wl.rec[0, 2]          # duplicate receiver cell
    wl.rec[1, 4] = wl.src[1, 0]          # receiver on a source cell
    wl.rec[2, 0] = -1
    one = run_gpu(wl, snap=snap, ckpt_every=ckpt, time_block=1)
    two = run_gpu(wl, snap=snap, ckpt_every=ckpt, time_block=2)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(two[key], one[key], err_msg=f"{key} order {order} {snap} K={ckpt}")


@pytest.mark.parametrize("order", inputs.ORDERS)
@pytest.mark.parametrize("snap,ckpt", [("f32", 0), ("bf16", 0), ("fp8", 0), ("f32", 7)])
def test_uniform_cq_two_step_bitwise_equals_single_steps(order, snap, ckpt):
    """mu_r one value everywhere: the two-step kernels read no Cq bytes and
    use the value instead, the one-step kernels read the array; both give
    bitwise the same records and gradients (the one-step kernels' FP8
    snapshots are checked against the oracle elsewhere)."""
    wl = inputs.as_f32(inputs.random_workload(order, 70, 9, nt=101, n_shots=3, n_src=3, n_rec=7,
                                              seed=830 + order, src_anywhere=True, mu_range=(1.0, 1.0)))
    assert np.all(wl.cq == wl.cq.flat[0])
    one = run_gpu(wl, snap=snap, ckpt_every=ckpt, time_block=1)
    two = run_gpu(wl, snap=snap, ckpt_every=ckpt, time_block=2)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(two[key], one[key], err_msg=f"{key} order {order} {snap} K={ckpt}")


@pytest.mark.parametrize("snap", ["f32", "bf16"])
def test_uniform_cq_host_storage_and_step_ratio_bitwise(snap):
    """mu_r one value: the Cq-free instances with snapshots in pinned host
    memory equal the device store bitwise, and with a snapshot step ratio of
    2 two steps per launch equal one step per launch bitwise."""
    wl = inputs.as_f32(inputs.random_workload(8, 48, 8, nt=41, n_shots=2, n_src=2, n_rec=5, seed=870,
                                              src_anywhere=True, mu_range=(1.0, 1.0)))
    dev = run_gpu(wl, snap=snap)
    host = run_gpu(wl, snap=snap, storage=1)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(host[key], dev[key], err_msg=f"host store {snap} {key}")
    one = run_gpu(wl, snap=snap, step_ratio=2, time_block=1)
    two = run_gpu(wl, snap=snap, step_ratio=2, time_block=2)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(two[key], one[key], err_msg=f"step ratio 2 {snap} {key}")


def test_uniform_cq_selects_the_cq_free_instances():
    """With TM_FWD_CHECK a forward over a uniform Cq runs the instances that
    read no Cq (timed as k_fwd_step2_uq), and so do the adjoint
    (k_adj_step2_uq) and its checkpoint replays given the same cq pointer;
    without the check, with a non-uniform Cq, or with another cq pointer
    (same values) for the adjoint, the array instances run."""
    import torch

    from tm_maxwell_fdtd_amd import native

    def counts(wl, check, ckpt_every=0, other_cq=False):
        prop = native.Propagator(wl, ckpt_every=ckpt_every, time_block=2)   # (not the resident kernels)
        try:
            native.tm_timing_enable(prop.plan, 1)
            r = prop.forward(store=True, check=check)
            _, fwd = native.tm_timing_read(prop.plan)
            if other_cq:
                prop.cq = prop.cq.clone()
            prop.adjoint(r)
            torch.cuda.synchronize()
            _, adj = native.tm_timing_read(prop.plan)
            native.tm_timing_enable(prop.plan, 0)
        finally:
            prop.close()
        # storing launches are timed apart ("_store"): full store mode stores
        # in tm_forward, checkpoint mode in the adjoint's replays only
        stored_fwd = {k for k, (_, n) in fwd.items() if n and k.endswith("_store")}
        stored_adj = {k for k, (_, n) in adj.items() if n and k.endswith("_store")}
        assert (stored_fwd == set()) == (ckpt_every > 0), (ckpt_every, fwd)
        assert (stored_adj != set()) == (ckpt_every > 0), (ckpt_every, adj)
        assert all(not k.startswith("k_fwd") or k.endswith("_store")
                   for k, (_, n) in fwd.items() if n and ckpt_every == 0), fwd

        def merged(d):
            out = {}
            for k, (_, n) in d.items():
                if n:
                    key = k[:-len("_store")] if k.endswith("_store") else k
                    out[key] = out.get(key, 0) + n
            return out
        return merged(fwd), merged(adj)

    uni = inputs.as_f32(inputs.random_workload(8, 40, 8, nt=40, n_shots=2, n_src=1, n_rec=4, seed=840,
                                               mu_range=(1.0, 1.0)))
    het = inputs.as_f32(inputs.random_workload(8, 40, 8, nt=40, n_shots=2, n_src=1, n_rec=4, seed=840))
    fwd, _ = counts(uni, check=True)
    assert fwd.get("k_fwd_step2_uq", 0) > 0 and "k_fwd_step2" not in fwd, fwd
    fwd, _ = counts(uni, check=False)
    assert fwd.get("k_fwd_step2", 0) > 0 and "k_fwd_step2_uq" not in fwd, fwd
    fwd, _ = counts(het, check=True)
    assert fwd.get("k_fwd_step2", 0) > 0 and "k_fwd_step2_uq" not in fwd, fwd
    fwd, adj = counts(uni, check=True, ckpt_every=8)
    assert fwd.get("k_fwd_step2_uq", 0) > 0 and "k_fwd_step2" not in fwd, fwd
    assert adj.get("k_fwd_step2_uq", 0) > 0 and "k_fwd_step2" not in adj, adj
    assert adj.get("k_adj_step2_uq", 0) > 0 and "k_adj_step2" not in adj, adj
    _, adj = counts(uni, check=True)
    assert adj.get("k_adj_step2_uq", 0) > 0 and "k_adj_step2" not in adj, adj
    for kw in (dict(check=True, other_cq=True), dict(check=False)):
        _, adj = counts(uni, ckpt_every=8, **kw)
        assert adj.get("k_fwd_step2", 0) > 0 and "k_fwd_step2_uq" not in adj, (kw, adj)
        assert adj.get("k_adj_step2", 0) > 0 and "k_adj_step2_uq" not in adj, (kw, adj)
    _, adj = counts(het, check=True)
    assert adj.get("k_adj_step2", 0) > 0 and "k_adj_step2_uq" not in adj, adj


@pytest.mark.parametrize("where", ["first", "interior", "last-used"])
def test_cq_one_differing_cell_is_not_uniform(orc, where):
    """Cq uniform except at one cell: the first cell (a halo cell the step
    never reads, but the reference value of the uniformity test), an
    interior cell, or the last cell any update reads.  The result must be
    that of the array, against the oracle and bitwise across launch shapes."""
    order = 4
    wl = inputs.as_f32(inputs.random_workload(order, 48, 8, nt=80, n_shots=2, n_src=2, n_rec=6,
                                              seed=850, mu_range=(1.0, 1.0)))
    p = order // 2
    cell = {"first": (0, 0), "interior": (wl.ny // 2 + 3, wl.nx // 2 - 5),
            "last-used": (wl.ny - p - 1, wl.nx - p - 1)}[where]
    wl.cq = wl.cq.copy()
    wl.cq[cell] = np.float64(np.float32(wl.cq[cell] * 1.5))
    got, _ = check(orc, wl, snap="f32", label=f"Cq differs at {where} {cell}")
    one = run_gpu(wl, snap="f32", grad_r=got["residual"], time_block=1)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=f"{key}: two-step != one-step ({where})")


def test_per_shot_models_uniform_cq_except_one_shot(orc):
    """Per-shot models, mu_r = 1 in every shot but one cell of the last
    shot's Cq: every shot against the oracle on its own model."""
    base = inputs.random_workload(4, 36, 8, nt=50, n_shots=3, n_src=2, n_rec=5, seed=860, mu_range=(1.0, 1.0))
    wl = inputs.as_f32(inputs.per_shot_models(base))
    wl.cq = wl.cq.copy()
    wl.cq[2, wl.ny // 2, wl.nx // 2] = np.float64(np.float32(wl.cq[2, wl.ny // 2, wl.nx // 2] * 0.75))
    refs = [orc.misfit_and_gradient(_shot_workload(wl, s)) for s in range(wl.n_shots)]
    resid = np.concatenate([ref["residual"] for ref in refs], axis=1)
    got = run_gpu(wl, snap="f32", grad_r=resid)
    for s, ref in enumerate(refs):
        e_r = rel_l2(got["records"][:, s], ref["records"][:, 0])
        e_g = max(rel_l2(got["gca_shot"][s], ref["gca_shot"][0]), rel_l2(got["gcb_shot"][s], ref["gcb_shot"][0]))
        print(f"[per-shot uniform Cq but one cell, shot {s}] records {e_r:.2e}  grads {e_g:.2e}", flush=True)
        assert e_r <= REC_TOL and e_g <= GRAD_TOL["f32"]


@pytest.mark.parametrize("npml,n_int", [(9, 300), (30, 60), (9, 40)])
def test_order8_forward_fifo_layouts_bitwise(npml, n_int):
    """Order 8: the two-step forward keeps stage A's x-band memories in
    compact FIFOs when every strip has at most 56 x-band lanes (one band of
    13 lanes per strip at 9 CPML cells and 316 columns; both bands, 26 lanes,
    in one strip at 40 interior columns) and in full FIFOs otherwise (both
    bands, 69 lanes, at 30 CPML cells and 128 columns).  Both give bitwise
    the results of one step per launch."""
    wl = inputs.as_f32(inputs.random_workload(8, 40, npml, nt=37, n_shots=2, n_src=2, n_rec=5, seed=880 + npml,
                                              src_anywhere=True, nx_int=n_int, mu_range=(1.0, 1.0)))
    for snap in ("bf16", "f32"):
        one = run_gpu(wl, snap=snap, time_block=1)
        two = run_gpu(wl, snap=snap, time_block=2)
        for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
            np.testing.assert_array_equal(two[key], one[key], err_msg=f"{key} npml {npml} nx_int {n_int} {snap}")


@pytest.mark.parametrize("steps,ckpt,chunks", [(1, 0, None), (3, 0, None), (8, 0, [5, 50]), (3, 7, None),
                                               (5, 0, [33])])
def test_event_blocks_bitwise(monkeypatch, steps, ckpt, chunks):
    """Sources and receivers go through event rows prepared for runs of
    steps; short runs (one step, odd lengths that split pairs, a run
    boundary inside a forward chunk or a checkpoint segment) give bitwise the
    records and gradients of one run for the whole problem."""
    wl = inputs.as_f32(inputs.random_workload(8, 40, 8, nt=61, n_shots=3, n_src=3, n_rec=7, seed=740,
                                              src_anywhere=True))
    wl.src[1, 1] = wl.src[1, 0]
    wl.src[2, 2] = -1
    wl.rec[0, 3] = wl.rec[0, 2]
    wl.rec[1, 4] = wl.src[1, 0]
    wl.rec[2, 0] = -1
    ref = run_gpu(wl, snap="f32", ckpt_every=ckpt)
    monkeypatch.setenv("TM_FDTD_EVENT_STEPS", str(steps))
    got = run_gpu(wl, snap="f32", ckpt_every=ckpt, chunks=chunks)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{key} steps {steps} K={ckpt} {chunks}")
    assert np.all(got["records"][:, 2, 0] == 0) and np.all(got["grad_f"][:, 2, 2] == 0)   # absent entries


def test_error_codes_on_device():
    import torch

    from tm_maxwell_fdtd_amd import native

    wl = inputs.as_f32(inputs.make_config(1, nt=20))
    prop = native.Propagator(wl)
    try:
        # adjoint with gradients before any storing forward
        with pytest.raises(native.TmError) as ei:
            prop.adjoint(torch.zeros((wl.nt, 1, wl.n_rec), device=prop.device))
        assert ei.value.status == native.TM_ESTATE
        prop.forward(store=False)
        with pytest.raises(native.TmError) as ei:
            prop.adjoint(torch.zeros((wl.nt, 1, wl.n_rec), device=prop.device))
        assert ei.value.status == native.TM_ESTATE
        # continuing a chunk from the wrong step
        with pytest.raises(native.TmError) as ei:
            prop.forward(t0=5, t1=10)
        assert ei.value.status == native.TM_ESTATE
        # workspace too small
        st = native.tm_forward(prop.plan, native.ptr(prop.ws), prop.ws_bytes - 256, native.ptr(prop.ca),
                               native.ptr(prop.cb), native.ptr(prop.cq), native.ptr(prop.f), None, 0, 5, 0,
                               native.stream_handle())
        assert st == native.TM_ENOMEM
        # unstable model: Courant number above 1
        assert prop.courant() == pytest.approx(0.9, rel=1e-5)
        prop.cb.mul_(1.5)
        with pytest.raises(native.TmError) as ei:
            prop.forward(check=True)
        assert ei.value.status == native.TM_EUNSTABLE
    finally:
        prop.close()



@pytest.mark.parametrize("order", inputs.ORDERS)
def test_grad_eps_sigma(orc, order):
    """tm_grad_eps_sigma against the oracle's chain rule, on the GPU's own
    dJ/dCa, dJ/dCb (isolates the chain rule) and end to end (the oracle's
    fp64 gradients through the oracle's chain rule)."""
    import torch

    from tm_maxwell_fdtd_amd import native

    wl = inputs.as_f32(inputs.random_workload(order, 40, 8, nt=120, n_shots=2, n_src=1, n_rec=7,
                                              seed=500 + order, sig_range=(0.0, 0.04)))
    ref = run_oracle(orc, wl)
    prop = native.Propagator(wl)
    try:
        r = prop.forward(store=True)
        resid = torch.as_tensor(np.asarray(ref["residual"], np.float32), device=prop.device)
        _, gca_s, gcb_s = prop.adjoint(resid)
        gca, gcb = prop.grad(gca_s, gcb_s)
        geps, gsig = prop.grad_eps_sigma(gca, gcb)
        # a null output is skipped, a null input counts as zero
        geps_a, gsig_a = prop.grad_eps_sigma(gca, None)
        st = native.tm_grad_eps_sigma(prop.plan, native.ptr(prop.ca), native.ptr(prop.cb), native.ptr(gca),
                                      native.ptr(gcb), 0.0, native.ptr(geps_a), None, native.stream_handle())
        assert st == native.TM_EINVAL
        torch.cuda.synchronize()
        g_ca, g_cb = gca.cpu().numpy().astype(np.float64), gcb.cpu().numpy().astype(np.float64)
        got_e, got_s = geps.cpu().numpy(), gsig.cpu().numpy()
        got_ea, got_sa = geps_a.cpu().numpy(), gsig_a.cpu().numpy()
        del r
    finally:
        prop.close()
    # the chain rule alone, on identical float32 inputs
    ce, cs = orc.eps_sigma_grad(wl.eps_r, wl.sigma, wl.dt, g_ca, g_cb)
    e1, s1 = rel_l2(got_e, ce), rel_l2(got_s, cs)
    ce_a, cs_a = orc.eps_sigma_grad(wl.eps_r, wl.sigma, wl.dt, g_ca, np.zeros_like(g_cb))
    e2, s2 = rel_l2(got_ea, ce_a), rel_l2(got_sa, cs_a)
    # end to end against the oracle's gradients
    oe, os_ = orc.eps_sigma_grad(wl.eps_r, wl.sigma, wl.dt, ref["gca"], ref["gcb"])
    e3, s3 = rel_l2(got_e, oe), rel_l2(got_s, os_)
    print(f"[eps/sigma o{order}] chain rule {e1:.2e} {s1:.2e}  (Cb input null) {e2:.2e} {s2:.2e}  "
          f"end to end {e3:.2e} {s3:.2e}", flush=True)
    assert max(e1, s1, e2, s2) <= 1e-5
    assert max(e3, s3) <= GRAD_TOL["f32"]
    mask = np.zeros((wl.ny, wl.nx), bool)
    mask[wl.pml_y0:wl.pml_y1, wl.pml_x0:wl.pml_x1] = True
    assert not np.any(got_e[~mask]) and not np.any(got_s[~mask])


def test_fp8_conversion_matches_oracle(orc):
    """tm_fp8_encode / tm_fp8_decode (the conversions of the FP8 snapshot
    store) against the oracle's encoder written from the E4M3 format."""
    import torch

    from tm_maxwell_fdtd_amd import native

    vals = [orc.e4m3_decode(c) for c in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    rng = np.random.default_rng(9)
    x = np.concatenate([
        np.float32(vals), -np.float32(vals), np.float32(mids), -np.float32(mids),
        np.nextafter(np.float32(mids), np.float32(0)), np.nextafter(np.float32(mids), np.float32(1e9)),
        np.float32([448.0, 449.0, 464.0, 1e5, -1e30, np.inf, -np.inf, 2.0 ** -10, 2.0 ** -11, -0.0]),
        (2.0 ** rng.uniform(-14, 10, 20000) * rng.choice([-1, 1], 20000)).astype(np.float32),
    ]).astype(np.float32)
    dev = torch.device("cuda")
    xin = torch.from_numpy(x).to(dev)
    codes = torch.empty(x.size, dtype=torch.uint8, device=dev)
    assert native.tm_fp8_encode(native.ptr(xin), native.ptr(codes), x.size, native.stream_handle()) == 0
    allc = torch.arange(256, dtype=torch.int32).to(torch.uint8).to(dev)
    dec = torch.empty(256, dtype=torch.float32, device=dev)
    assert native.tm_fp8_decode(native.ptr(allc), native.ptr(dec), 256, native.stream_handle()) == 0
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    ref = np.array([orc.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:10]]
    d = dec.cpu().numpy().astype(np.float64)
    r = np.array([orc.e4m3_decode(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(d), np.isnan(r))
    np.testing.assert_array_equal(d[~np.isnan(d)], r[~np.isnan(r)])
    # a NaN input stays NaN
    nan = torch.full((4,), float("nan"), device=dev)
    c4 = torch.empty(4, dtype=torch.uint8, device=dev)
    assert native.tm_fp8_encode(native.ptr(nan), native.ptr(c4), 4, native.stream_handle()) == 0
    assert all((int(v) & 0x7F) == 0x7F for v in c4.cpu().numpy())


@pytest.mark.parametrize("order", inputs.ORDERS)
def test_fp8_snapshots(orc, order):
    """FP8 E4M3 snapshots against the oracle's adjoint of the same quantized
    snapshots (the oracle quantizes its float32-rounded values, as the kernels
    do)."""
    wl = inputs.as_f32(inputs.random_workload(order, 60, 8, nt=140, n_shots=2, n_src=1, n_rec=9,
                                              seed=220 + order))
    ref = orc.misfit_and_gradient(wl, snap_quant="fp8")
    got = run_gpu(wl, snap="fp8", grad_r=ref["residual"])
    e_r = rel_l2(got["records"], ref["records"])
    e_a = rel_l2(got["gca_shot"], ref["gca_shot"])
    e_b = rel_l2(got["gcb_shot"], ref["gcb_shot"])
    e_f = rel_l2(got["grad_f"], ref["grad_f"])
    exact = orc.misfit_and_gradient(wl)
    q_a = rel_l2(ref["gca_shot"], exact["gca_shot"])
    print(f"[fp8-o{order}] records {e_r:.2e}  gCa {e_a:.2e}  gCb {e_b:.2e}  grad_f {e_f:.2e}  "
          f"(fp8 vs exact snapshots in the oracle: gCa {q_a:.2e})", flush=True)
    assert e_r <= REC_TOL and e_f <= GRAD_TOL["f32"]
    assert e_a <= FP8_TOL and e_b <= FP8_TOL


@pytest.mark.parametrize("snap", ["f32", "bf16", "fp8"])
def test_host_storage_bitwise_equals_device_storage(snap):
    """Snapshots kept in pinned host memory through a ring of device slots
    give bitwise the results of the device store (one and two steps per
    launch, whole and chunked forward)."""
    wl = inputs.as_f32(inputs.random_workload(8, 60, 8, nt=47, n_shots=2, n_src=2, n_rec=6, seed=730,
                                              src_anywhere=True))
    dev = run_gpu(wl, snap=snap)
    for tb, chunks in ((2, None), (1, None), (2, [13, 30])):
        host = run_gpu(wl, snap=snap, storage=1, time_block=tb, chunks=chunks)
        for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
            np.testing.assert_array_equal(host[key], dev[key], err_msg=f"{snap} time_block {tb} {chunks} {key}")


@pytest.mark.parametrize("ratio,storage", [(2, 0), (3, 0), (3, 1), (5, 1)])
def test_step_ratio(orc, ratio, storage):
    """Snapshots every R-th step, gradient terms weighted by R, against the
    oracle's gradient of the same subsampled store; R = 1 is checked by every
    other test."""
    wl = inputs.as_f32(inputs.random_workload(4, 50, 8, nt=61, n_shots=2, n_src=1, n_rec=7, seed=740 + ratio))
    ref = orc.misfit_and_gradient(wl, step_ratio=ratio)
    got = run_gpu(wl, snap="f32", grad_r=ref["residual"], storage=storage, step_ratio=ratio)
    full = orc.misfit_and_gradient(wl)
    e_a, e_b = rel_l2(got["gca_shot"], ref["gca_shot"]), rel_l2(got["gcb_shot"], ref["gcb_shot"])
    e_r = rel_l2(got["records"], ref["records"])
    print(f"[step ratio {ratio}, storage {storage}] records {e_r:.2e}  gCa {e_a:.2e}  gCb {e_b:.2e}  "
          f"(subsampled vs full gradient in the oracle: {rel_l2(ref['gca'], full['gca']):.2e})", flush=True)
    assert e_r <= REC_TOL
    assert e_a <= GRAD_TOL["f32"] and e_b <= GRAD_TOL["f32"]


@pytest.mark.parametrize("ratio,storage", [(2, 0), (3, 0), (3, 1)])
def test_step_ratio_two_step_launch_bitwise(ratio, storage):
    """With a snapshot step ratio a pair of adjoint steps may hold one stored
    step or none; two steps per launch still give bitwise the results of one
    step per launch (host storage runs the adjoint one step per launch)."""
    wl = inputs.as_f32(inputs.random_workload(8, 40, 8, nt=37, n_shots=2, n_src=2, n_rec=5, seed=770 + ratio,
                                              src_anywhere=True))
    one = run_gpu(wl, snap="bf16", storage=storage, step_ratio=ratio, time_block=1)
    two = run_gpu(wl, snap="bf16", storage=storage, step_ratio=ratio, time_block=2)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(two[key], one[key], err_msg=f"{key} R={ratio} storage {storage}")


def _shot_workload(wl, s):
    """Shot s of a workload with one model per shot, as a one-shot workload
    with that shot's model (shots are independent)."""
    import dataclasses

    from gpu_util import sub_workload

    return dataclasses.replace(sub_workload(wl, [s]), ca=wl.ca[s].copy(), cb=wl.cb[s].copy(), cq=wl.cq[s].copy())


@pytest.mark.parametrize("order", inputs.ORDERS)
def test_per_shot_models(orc, order):
    """One model per shot (batched models): every shot's records, per-shot
    gradients and source gradient against the oracle run on that shot with
    its own model; one and two steps per launch bitwise equal."""
    base = inputs.random_workload(order, 40, 8, nt=60, n_shots=3, n_src=2, n_rec=6, seed=780 + order)
    wl = inputs.as_f32(inputs.per_shot_models(base))
    assert wl.ca.shape == (3, wl.ny, wl.nx)
    refs = [orc.misfit_and_gradient(_shot_workload(wl, s)) for s in range(wl.n_shots)]
    resid = np.concatenate([ref["residual"] for ref in refs], axis=1)
    got = run_gpu(wl, snap="f32", grad_r=resid)
    one = run_gpu(wl, snap="f32", grad_r=resid, time_block=1)
    for s, ref in enumerate(refs):
        e = {"records": rel_l2(got["records"][:, s], ref["records"][:, 0]),
             "gca_shot": rel_l2(got["gca_shot"][s], ref["gca_shot"][0]),
             "gcb_shot": rel_l2(got["gcb_shot"][s], ref["gcb_shot"][0]),
             "grad_f": rel_l2(got["grad_f"][:, s], ref["grad_f"][:, 0])}
        print(f"[per-shot models o{order} shot {s}] " + "  ".join(f"{k} {v:.2e}" for k, v in e.items()), flush=True)
        assert e["records"] <= REC_TOL
        assert max(e["gca_shot"], e["gcb_shot"], e["grad_f"]) <= GRAD_TOL["f32"]
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=f"{key}: two-step != one-step")


def test_per_shot_models_identical_equal_shared_model():
    """S identical per-shot models give bitwise the results of the shared model."""
    import dataclasses

    wl = inputs.as_f32(inputs.random_workload(8, 40, 8, nt=40, n_shots=3, n_src=2, n_rec=5, seed=790))
    rep = dataclasses.replace(wl, ca=np.stack([wl.ca] * 3), cb=np.stack([wl.cb] * 3), cq=np.stack([wl.cq] * 3))
    a, b = run_gpu(wl, snap="bf16"), run_gpu(rep, snap="bf16")
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(b[key], a[key], err_msg=key)


def test_per_shot_models_eps_sigma_and_courant(orc):
    """The chain rule to eps_r / sigma per shot at each shot's own model, and
    the Courant check over all shots' models."""
    import torch

    from tm_maxwell_fdtd_amd import native

    base = inputs.random_workload(4, 30, 8, nt=20, n_shots=3, n_src=1, n_rec=3, seed=795, sig_range=(0.0, 0.04))
    wl = inputs.as_f32(inputs.per_shot_models(base))
    prop = native.Propagator(wl)
    try:
        rng = np.random.default_rng(5)
        gca = torch.as_tensor(rng.standard_normal(wl.ca.shape).astype(np.float32), device=prop.device)
        gcb = torch.as_tensor(rng.standard_normal(wl.ca.shape).astype(np.float32), device=prop.device)
        geps, gsig = prop.grad_eps_sigma(gca, gcb)
        c_all = prop.courant()
        torch.cuda.synchronize()
        got_e, got_s = geps.cpu().numpy(), gsig.cpu().numpy()
        g_ca, g_cb = gca.cpu().numpy().astype(np.float64), gcb.cpu().numpy().astype(np.float64)
    finally:
        prop.close()
    S = wl.n_shots
    for s in range(S):
        eps_s = base.eps_r * (1.0 + 0.25 * s / (S - 1))
        ce, cs = orc.eps_sigma_grad(eps_s, base.sigma, wl.dt, g_ca[s], g_cb[s])
        assert rel_l2(got_e[s], ce) <= 1e-5 and rel_l2(got_s[s], cs) <= 1e-5, s
    # the fastest model is shot 0's (the smallest eps_r): its Courant number
    shot0 = native.Propagator(_shot_workload(wl, 0))
    try:
        c0 = shot0.courant()
    finally:
        shot0.close()
    assert c_all == pytest.approx(c0, rel=1e-6)


@pytest.mark.parametrize("mode", ["ckpt", "host"])
def test_per_shot_models_storage_modes(mode):
    """One model per shot with checkpoint replay (the replay reads every
    shot's own model again) or with the pinned-host snapshot store: bitwise
    the results of the full device store."""
    base = inputs.random_workload(4, 36, 8, nt=45, n_shots=3, n_src=2, n_rec=5, seed=800)
    wl = inputs.as_f32(inputs.per_shot_models(base))
    ref = run_gpu(wl, snap="f32", ckpt_every=0)
    kw = dict(ckpt_every=9) if mode == "ckpt" else dict(ckpt_every=0, storage=1)
    got = run_gpu(wl, snap="f32", **kw)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{mode} {key}")


@pytest.mark.parametrize("order", [4, 8])
def test_event_rows_everywhere(orc, order):
    """A receiver line down a column (an event row on every row of the E set)
    and sources on many rows: every block runs the general iteration, the
    event rows span the whole window; against the oracle, and one and two
    steps per launch bitwise equal."""
    wl = inputs.random_workload(order, 40, 8, nt=40, n_shots=2, n_src=6, n_rec=8, seed=820 + order,
                                src_anywhere=True)
    p = order // 2
    rows = np.arange(p, wl.ny - p + 1)
    wl.rec = np.stack([rows * wl.nx + (wl.nx // 2 + s) for s in range(2)]).astype(np.int64)   # [S][n_rec]
    rng = np.random.default_rng(821)
    wl.src = np.stack([rng.choice(rows, 6) * wl.nx + (p + 3 * s + 1) for s in range(2)]).astype(np.int64)
    wl.f = wl.f[:, :, :1].repeat(6, axis=2)
    wl = inputs.as_f32(wl)
    ref = run_oracle(orc, wl)
    got = run_gpu(wl, snap="f32", grad_r=ref["residual"])
    one = run_gpu(wl, snap="f32", grad_r=ref["residual"], time_block=1)
    regions = grid_regions(wl)
    tol = GRAD_TOL["f32"]
    errs = {k: compare(k, got[k], ref[k], t, regions if k.startswith("gc") else None)
            for k, t in (("records", REC_TOL), ("gca_shot", tol), ("gcb_shot", tol), ("grad_f", tol))}
    print(f"[events everywhere o{order}] n_rec {wl.n_rec}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()),
          flush=True)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=key)


# ---------------------------------------------------------------------------
# CPML coordinate stretching (kappa != 1) and the band flags, on the GPU
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("order", inputs.ORDERS)
@pytest.mark.parametrize("snap,ckpt,tb,mu", [("f32", 0, 2, 2.0), ("f32", 0, 1, 2.0), ("bf16", 0, 2, 2.0),
                                             ("f32", 7, 2, 2.0), ("f32", 7, 1, 2.0), ("f32", 0, 2, 1.0),
                                             ("bf16", 7, 2, 1.0)])
def test_stretched_cpml(orc, order, snap, ckpt, tb, mu):
    """kappa rising from 1 to 5 into every band (the d / kappa terms of all
    four forward filters and their adjoints run with kappa != 1 on every
    band cell), heterogeneous model, sources and receivers in the bands too;
    one and two steps per launch, fp32 and bf16 snapshots, checkpointing,
    and mu_r = 1 (the instances that take Cq as one value)."""
    wl = inputs.random_workload(order, 44, 9, nt=90, n_shots=2, n_src=3, n_rec=6, seed=700 + order,
                                src_anywhere=True, kappa_max=5.0, mu_range=(1.0, mu))
    wl = inputs.as_f32(wl)
    assert np.all(wl.cpml[2, order // 2:wl.pml_y0] > 1.0)
    check(orc, wl, snap=snap, ckpt_every=ckpt, time_block=tb,
          label=f"kappa-o{order}-{snap}-K{ckpt}-tb{tb}-mu{mu:g}")


@pytest.mark.parametrize("order", inputs.ORDERS)
@pytest.mark.parametrize("tb", [3, 1, 2])
def test_cpml_probe_sites_and_flags(orc, order, tb):
    """The oracle's closed-form CPML probe (one filter site at one index,
    tests/cpml_probe.py) through the C ABI: every site at lo-1, lo, hi-2,
    hi-1 and hi, kappa 1.7 and 4, records against the oracle and against the
    closed form; time_block 3 runs the resident small-grid kernels."""
    import cpml_probe

    from tm_maxwell_fdtd_amd import native
    import torch

    c1 = float(orc.coefficients(order)[0])
    for kappa in (1.7, 4.0):
        for site, where in cpml_probe.CASES:
            wl, info = cpml_probe.workload(order, site, where, kappa, seed=900 + order)
            ref, _, _ = orc.forward(wl)
            prop = native.Propagator(wl, time_block=tb)
            try:
                r = prop.forward(store=False)
                torch.cuda.synchronize()
                got = r.cpu().numpy()
            finally:
                prop.close()
            exp = cpml_probe.expected_records(wl, info, c1)
            e_o = rel_l2(got[:, 0, 0], ref[:, 0, 0])
            e_c = float(np.abs(got[:, 0, 0] - exp).max() / np.abs(exp).max())
            assert e_o <= REC_TOL and e_c <= 1e-5, (site, where, kappa, e_o, e_c)


def test_set_indices_equals_a_fresh_plan(orc):
    """A plan re-pointed at a new acquisition geometry with
    tm_plan_set_indices (more event rows: a larger workspace) gives bitwise
    the results of a plan created with that geometry, and those match the
    oracle; the adjoint right after the switch is refused (TM_ESTATE)."""
    import dataclasses

    import torch

    from tm_maxwell_fdtd_amd import native

    wa = inputs.as_f32(inputs.random_workload(8, 50, 8, nt=60, n_shots=2, n_src=2, n_rec=6, seed=870))
    rng = np.random.default_rng(871)
    ys = rng.integers(wa.pml_y0 - 4, wa.pml_y1 + 4, size=(2, 6))
    xs = rng.integers(wa.pml_x0, wa.pml_x1, size=(2, 6))
    rec_b = (ys * wa.nx + xs).astype(np.int64)
    wb = dataclasses.replace(wa, rec=rec_b)
    fresh = run_gpu(wb, snap="f32")
    prop = native.Propagator(wa)
    try:
        r = prop.forward(store=True)
        prop.adjoint(r)
        bytes_a = prop.ws_bytes
        prop.set_indices(wb.src, wb.rec)
        assert prop.ws_bytes >= bytes_a
        with pytest.raises(native.TmError) as ei:
            prop.adjoint(r)
        assert ei.value.status == native.TM_ESTATE
        r = prop.forward(store=True)
        grad_f, gca, gcb = prop.adjoint(r)
        torch.cuda.synchronize()
        got = dict(records=r.cpu().numpy(), grad_f=grad_f.cpu().numpy(), gca_shot=gca.cpu().numpy(),
                   gcb_shot=gcb.cpu().numpy())
    finally:
        prop.close()
    for key in ("records", "grad_f", "gca_shot", "gcb_shot"):
        np.testing.assert_array_equal(got[key], fresh[key], err_msg=key)
    ref = run_oracle(orc, wb)
    compare("records", got["records"], ref["records"], REC_TOL)
    compare("gCa/shot", got["gca_shot"], ref["gca_shot"], GRAD_TOL["f32"], grid_regions(wb))


# ---------------------------------------------------------------------------
# Resident kernels for small grids (the whole shot in one workgroup's LDS)
# ---------------------------------------------------------------------------

def _kernel_counts(wl, **kw):
    """Run forward (storing) + adjoint with timing on; the kernels that ran."""
    import torch

    from tm_maxwell_fdtd_amd import native

    prop = native.Propagator(wl, **kw)
    try:
        native.tm_timing_enable(prop.plan, 1)
        r = prop.forward(store=True)
        prop.adjoint(r)
        torch.cuda.synchronize()
        _, kt = native.tm_timing_read(prop.plan)
        native.tm_timing_enable(prop.plan, 0)
    finally:
        prop.close()
    return {k for k, (_, n) in kt.items() if n}


@pytest.mark.parametrize("order", inputs.ORDERS)
@pytest.mark.parametrize("snap,ratio,kappa", [("f32", 1, 1.0), ("bf16", 1, 4.0), ("fp8", 1, 1.0), ("f32", 3, 4.0)])
def test_resident_small_grid_bitwise(orc, order, snap, ratio, kappa):
    """A grid that fits one workgroup's LDS runs the resident kernels with
    time_block 3: bitwise the records, per-shot gradients and grad_f of one
    step per launch, and the oracle's within the tolerances.
    Sources and receivers anywhere (bands, edge rows), duplicates and
    negative indices, stretched CPML, snapshot kinds and step ratios."""
    wl = inputs.random_workload(order, 40, 7, nt=57, n_shots=3, n_src=3, n_rec=6, seed=1300 + order,
                                src_anywhere=True, kappa_max=kappa)
    wl.src[1, 1] = wl.src[1, 0]
    wl.src[2, 2] = -1
    wl.rec[0, 3] = wl.rec[0, 2]
    wl.rec[2, 0] = -1
    wl.rec[1, 4] = wl.src[1, 0]
    wl = inputs.as_f32(wl)
    assert wl.ny * wl.nx <= 8192
    ran = _kernel_counts(wl, snap=snap, step_ratio=ratio, time_block=3)
    assert "k_adj_small" in ran and any(k.startswith("k_fwd_small") for k in ran), ran
    assert not any(k.startswith(("k_fwd_step", "k_adj_step")) for k in ran), ran
    got = run_gpu(wl, snap=snap, step_ratio=ratio, time_block=3)
    one = run_gpu(wl, snap=snap, step_ratio=ratio, time_block=1)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=key)
    if snap == "f32":
        ref = orc.misfit_and_gradient(wl, step_ratio=ratio)
        regions = grid_regions(wl)
        compare("records", got["records"], ref["records"], REC_TOL)
        compare("gCa/shot", got["gca_shot"], ref["gca_shot"], GRAD_TOL["f32"], regions)
        compare("gCb/shot", got["gcb_shot"], ref["gcb_shot"], GRAD_TOL["f32"], regions)
        compare("grad_f", got["grad_f"], ref["grad_f"], GRAD_TOL["f32"])


@pytest.mark.parametrize("case", ["chunks", "event-blocks", "per-shot-models", "no-grads", "ckpt-plan"])
def test_resident_small_grid_modes(monkeypatch, case):
    """The resident kernels under the other call patterns, bitwise against
    one step per launch: forward chunks (the state crosses launches), short
    event blocks (one launch per block), one model per shot, an adjoint
    without gradients, and a checkpointing plan (its storing forward and
    replays stream, its gradient-free calls may run resident)."""
    import torch

    from tm_maxwell_fdtd_amd import native

    wl = inputs.as_f32(inputs.random_workload(4, 40, 7, nt=41, n_shots=2, n_src=2, n_rec=5, seed=1320,
                                              src_anywhere=True, kappa_max=3.0))
    kw, chunks = {}, None
    if case == "chunks":
        chunks = [7, 8, 30]
    elif case == "event-blocks":
        monkeypatch.setenv("TM_FDTD_EVENT_STEPS", "6")
    elif case == "per-shot-models":
        wl = inputs.as_f32(inputs.per_shot_models(wl))
    elif case == "ckpt-plan":
        kw = dict(ckpt_every=9)
    if case == "no-grads":
        outs = []
        for tb in (3, 1):
            prop = native.Propagator(wl, time_block=tb)
            try:
                r = prop.forward(store=False)
                d = torch.randn(r.shape, generator=torch.Generator().manual_seed(5)).to(prop.device)
                gf, _, _ = prop.adjoint(d, want_grads=False)
                torch.cuda.synchronize()
                outs.append((r.cpu().numpy(), gf.cpu().numpy()))
            finally:
                prop.close()
        np.testing.assert_array_equal(outs[0][0], outs[1][0])
        np.testing.assert_array_equal(outs[0][1], outs[1][1])
        return
    got = run_gpu(wl, snap="f32", chunks=chunks, time_block=3, **kw)
    one = run_gpu(wl, snap="f32", chunks=chunks, time_block=1, **kw)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=f"{case} {key}")


BAND_KERNELS = {4: "k_adj_band", 5: "k_adj_bandk"}


@pytest.mark.parametrize("tb", [4, 5])
@pytest.mark.parametrize("order", inputs.ORDERS)
@pytest.mark.parametrize("snap,ratio,kappa", [("f32", 1, 1.0), ("bf16", 1, 4.0), ("fp8", 1, 1.0), ("f32", 3, 4.0)])
def test_banded_small_grid_bitwise(order, snap, ratio, kappa, tb):
    """The banded resident kernels (time_block 4: several workgroups per
    shot, rows exchanged between neighbouring bands every step; time_block
    5: each band also steps 2(2P-1) rows of its neighbours and the bands
    exchange their whole state every second step) give bitwise the records,
    per-shot gradients and grad_f of the single-workgroup resident kernels
    and of one step per launch.  Sources and receivers anywhere (bands, edge
    rows, duplicates, negative indices), stretched CPML, snapshot kinds and
    step ratios."""
    wl = inputs.random_workload(order, 40, 7, nt=57, n_shots=3, n_src=3, n_rec=6, seed=1400 + order,
                                src_anywhere=True, kappa_max=kappa)
    wl.src[1, 1] = wl.src[1, 0]
    wl.src[2, 2] = -1
    wl.rec[0, 3] = wl.rec[0, 2]
    wl.rec[2, 0] = -1
    wl.rec[1, 4] = wl.src[1, 0]
    wl = inputs.as_f32(wl)
    ran = _kernel_counts(wl, snap=snap, step_ratio=ratio, time_block=tb)
    # (time_block 5 at order 8: 2 x 14 extended rows of 62 cells exceed the
    # 2048 cells of a blocked band, so the bands exchange every step)
    assert BAND_KERNELS[4 if order == 8 else tb] in ran and any(k.startswith("k_fwd_band") for k in ran), ran
    assert not any(k.startswith(("k_fwd_step", "k_adj_step", "k_fwd_small", "k_adj_small")) for k in ran), ran
    got = run_gpu(wl, snap=snap, step_ratio=ratio, time_block=tb)
    res = run_gpu(wl, snap=snap, step_ratio=ratio, time_block=3)
    one = run_gpu(wl, snap=snap, step_ratio=ratio, time_block=1)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], res[key], err_msg=f"resident {key}")
        np.testing.assert_array_equal(got[key], one[key], err_msg=f"one step {key}")
    assert np.abs(got["records"]).max() > 0


@pytest.mark.parametrize("tb", [4, 5])
@pytest.mark.parametrize("order,n_int,nx_int,shots", [(2, 150, 90, 1), (4, 120, 200, 2), (8, 60, 150, 4)])
def test_banded_larger_grid(orc, order, n_int, nx_int, shots, tb):
    """Grids too large for one workgroup's LDS, in bands: against one step
    per launch (bitwise) and the oracle (within the tolerances)."""
    wl = inputs.as_f32(inputs.random_workload(order, n_int, 8, nt=45, n_shots=shots, n_src=2, n_rec=8,
                                              seed=1420 + order, nx_int=nx_int))
    assert wl.ny * wl.nx > 8192
    ran = _kernel_counts(wl, time_block=tb)
    # (time_block 5 at orders 4 and 8: the extended rows of 220 and 174
    # cells exceed the 2048 cells of a blocked band, so the bands exchange
    # every step)
    assert BAND_KERNELS[tb if order == 2 else 4] in ran, ran
    got = run_gpu(wl, snap="f32", time_block=tb)
    one = run_gpu(wl, snap="f32", time_block=1)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=key)
    # (no per-region bounds: in 45 steps the fields reach some of the band
    # columns only as fp64 underflow-size values, which fp32 rounds to 0)
    ref = orc.misfit_and_gradient(wl)
    compare("records", got["records"], ref["records"], REC_TOL)
    compare("gCa/shot", got["gca_shot"], ref["gca_shot"], GRAD_TOL["f32"])
    compare("gCb/shot", got["gcb_shot"], ref["gcb_shot"], GRAD_TOL["f32"])
    compare("grad_f", got["grad_f"], ref["grad_f"], GRAD_TOL["f32"])


@pytest.mark.parametrize("tb", [4, 5])
@pytest.mark.parametrize("case", ["chunks", "event-blocks", "per-shot-models", "no-grads", "ckpt-plan"])
def test_banded_modes(monkeypatch, case, tb):
    """The banded kernels under the other call patterns, bitwise against
    one step per launch: forward chunks, short event blocks (one launch per
    block), one model per shot, an adjoint without gradients, and a
    checkpointing plan (its storing forward and replays stream)."""
    import torch

    from tm_maxwell_fdtd_amd import native

    wl = inputs.as_f32(inputs.random_workload(4, 60, 7, nt=41, n_shots=2, n_src=2, n_rec=5, seed=1440,
                                              src_anywhere=True, kappa_max=3.0))
    kw, chunks = {}, None
    if case == "chunks":
        chunks = [7, 8, 30]
    elif case == "event-blocks":
        monkeypatch.setenv("TM_FDTD_EVENT_STEPS", "6")
    elif case == "per-shot-models":
        wl = inputs.as_f32(inputs.per_shot_models(wl))
    elif case == "ckpt-plan":
        kw = dict(ckpt_every=9)
    if case == "no-grads":
        outs = []
        for b in (tb, 1):
            prop = native.Propagator(wl, time_block=b)
            try:
                r = prop.forward(store=False)
                d = torch.randn(r.shape, generator=torch.Generator().manual_seed(5)).to(prop.device)
                gf, _, _ = prop.adjoint(d, want_grads=False)
                torch.cuda.synchronize()
                outs.append((r.cpu().numpy(), gf.cpu().numpy()))
            finally:
                prop.close()
        np.testing.assert_array_equal(outs[0][0], outs[1][0])
        np.testing.assert_array_equal(outs[0][1], outs[1][1])
        return
    got = run_gpu(wl, snap="f32", chunks=chunks, time_block=tb, **kw)
    one = run_gpu(wl, snap="f32", chunks=chunks, time_block=1, **kw)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=f"{case} {key}")


def test_banded_kernels_by_default_for_small_problems():
    """time_block 0 runs the banded kernels on the small workloads (the
    order-2 86^2 grid with one shot: the blocked ones; the order-4 300^2
    grid with four: those exchanging every step) and the streaming kernels
    on a large one; bitwise equal to two steps per launch."""
    wl1 = inputs.as_f32(inputs.make_config(1, nt=30))
    wl2 = inputs.as_f32(inputs.make_config(2, nt=20))
    wl3 = inputs.as_f32(inputs.make_config(3, n_shots=1, nt=6))
    assert "k_adj_bandk" in _kernel_counts(wl1)
    assert "k_adj_band" in _kernel_counts(wl2)
    assert not any(k.startswith("k_adj_band") for k in _kernel_counts(wl3))
    for wl in (wl1, wl2):
        got = run_gpu(wl)
        two = run_gpu(wl, time_block=2)
        for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
            np.testing.assert_array_equal(got[key], two[key], err_msg=key)


@pytest.mark.parametrize("order,kx", [(2, 1), (2, 3), (2, 4), (4, 1), (8, 1)])
def test_blocked_banded_exchange_intervals(monkeypatch, order, kx):
    """The blocked banded kernels with other numbers of steps between
    exchanges (TM_FDTD_BAND_KX; the band heights follow), with an odd step
    count, so that the last run of steps between exchanges is short:
    bitwise one step per launch."""
    wl = inputs.random_workload(order, 70, 7, nt=47, n_shots=2, n_src=2, n_rec=6, seed=1470 + order + kx,
                                src_anywhere=True, kappa_max=3.0)
    wl = inputs.as_f32(wl)
    monkeypatch.setenv("TM_FDTD_BAND_KX", str(kx))
    ran = _kernel_counts(wl, time_block=5)
    assert "k_adj_bandk" in ran, ran
    got = run_gpu(wl, snap="bf16", step_ratio=2, time_block=5)
    monkeypatch.delenv("TM_FDTD_BAND_KX")
    one = run_gpu(wl, snap="bf16", step_ratio=2, time_block=1)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=key)


def test_blocked_banded_fewer_steps_where_three_do_not_fit():
    """An order-2 grid too wide for the extended rows of three steps between
    exchanges (9 rows of 265 cells > 2048) but not of two (6 rows): the
    blocked kernels still run, with two steps, bitwise one step per launch."""
    wl = inputs.as_f32(inputs.random_workload(2, 40, 8, nt=23, n_shots=1, n_src=2, n_rec=6, seed=1490,
                                              src_anywhere=True, nx_int=250))
    assert 9 * (wl.nx - 1) > 2048 >= 6 * (wl.nx - 1), wl.nx
    ran = _kernel_counts(wl, time_block=5)
    assert "k_adj_bandk" in ran and "k_adj_band" not in ran, ran
    got = run_gpu(wl, snap="f32", time_block=5)
    one = run_gpu(wl, snap="f32", time_block=1)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=key)


@pytest.mark.parametrize("tb", [4, 5])
def test_banded_failed_wait_is_reported(monkeypatch, tb):
    """A banded launch whose exchange wait fails (forced from the host with
    a poll limit of 0: every workgroup gives up at its first wait and leaves
    its time loop) makes tm_forward and tm_adjoint return TM_EHIP instead of
    hanging; the device stays usable and a plan without the forced failure
    gives the one-step-per-launch results."""
    from tm_maxwell_fdtd_amd import native

    wl = inputs.as_f32(inputs.random_workload(2, 60, 7, nt=20, n_shots=2, n_src=2, n_rec=4, seed=1460))
    monkeypatch.setenv("TM_FDTD_BAND_SPIN", "0")
    prop = native.Propagator(wl, time_block=tb)
    try:
        with pytest.raises(native.TmError) as e:
            prop.forward(store=True)
        assert e.value.status == native.TM_EHIP
    finally:
        prop.close()
    monkeypatch.delenv("TM_FDTD_BAND_SPIN")
    got = run_gpu(wl, snap="f32", time_block=tb)
    one = run_gpu(wl, snap="f32", time_block=1)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], one[key], err_msg=key)


@pytest.mark.parametrize("time_block", [2, 3, 4, 5])
def test_hip_graph_replays_bitwise(time_block):
    """The C-ABI calls of a forward with storage and an adjoint can be
    captured in a HIP graph (no host synchronisation, no memset nodes):
    every replay, with eager work on the stream between replays, gives
    bitwise the eager records, per-shot gradients and grad_f (streaming,
    single-workgroup resident, banded and blocked banded kernels)."""
    import torch

    from tm_maxwell_fdtd_amd import native

    wl = inputs.as_f32(inputs.random_workload(4, 40, 7, nt=33, n_shots=2, n_src=2, n_rec=5, seed=1480))
    prop = native.Propagator(wl, time_block=time_block)
    try:
        r = torch.zeros((wl.nt, wl.n_shots, wl.n_rec), dtype=torch.float32, device=prop.device)
        prop.forward(r=r, store=True, check=False)
        ref = [x.clone() for x in (r, *prop.adjoint(r))]
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):                   # warm-up on the capture stream
            prop.forward(r=r, store=True, check=False)
            prop.adjoint(r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            prop.forward(r=r, store=True, check=False)
            out = prop.adjoint(r)
        for i in range(3):
            junk = torch.randn(1 << 16, device=prop.device) * 3.0   # eager work between replays
            r.fill_(7.0)
            g.replay()
            torch.cuda.synchronize()
            for a, b, name in zip((r, *out), ref, ("records", "grad_f", "gca_shot", "gcb_shot")):
                assert torch.equal(a, b), f"replay {i}: {name}"
            del junk
    finally:
        prop.close()


def test_resident_kernels_by_default_from_16_shots():
    """time_block 0 picks the resident kernels for a grid that fits with 16
    shots or more, the streaming kernels with fewer; bitwise equal."""
    wl16 = inputs.as_f32(inputs.make_config(1, n_shots=16, nt=40))
    wl4 = inputs.as_f32(inputs.make_config(1, n_shots=4, nt=40))
    assert "k_adj_small" in _kernel_counts(wl16)
    assert "k_adj_small" not in _kernel_counts(wl4)
    got = run_gpu(wl16)
    two = run_gpu(wl16, time_block=2)
    for key in ("records", "gca_shot", "gcb_shot", "grad_f"):
        np.testing.assert_array_equal(got[key], two[key], err_msg=key)
