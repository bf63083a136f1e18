"""The C ABI on the CPU: the library loads, exports what the header declares,
and rejects invalid problems and call sequences on the host, before any HIP
call (no GPU is touched by these tests)."""

import ctypes

import numpy as np
import pytest

from tm_maxwell_fdtd_amd import inputs, native

from gpu_util import largest_square_grid

FAKE_WS = 1 << 20          # an aligned address never dereferenced by these calls


def make(wl, **over):
    d = native.make_desc(wl)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def create(wl, cpml=None, src="wl", rec="wl", **over):
    d = make(wl, **over)
    st, plan = native.tm_plan_create(d, wl.cpml if cpml is None else cpml,
                                     wl.src if isinstance(src, str) else src,
                                     wl.rec if isinstance(rec, str) else rec)
    if plan:
        native.tm_plan_destroy(plan)
    return st


@pytest.fixture(scope="module")
def wl():
    return inputs.make_config(2, n_int=40, nt=30, n_shots=2, n_rec=5)


def test_library_exports_every_declared_function():
    names = native.declared_functions()
    assert "tm_forward" in names and "tm_adjoint" in names and "tm_grad" in names
    lib = native.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_timed_kernel_names():
    """The timing ids name the step kernels; _uq marks the instances that
    use one Cq value instead of reading the array."""
    names = [native.tm_kernel_name(k) for k in range(native.tm_kernel_count())]
    assert names == ["k_fwd_step", "k_adj_step", "k_fwd_step2", "k_adj_step2", "k_fwd_step2_uq", "k_adj_step2_uq",
                     "k_fwd_step_store", "k_fwd_step2_store", "k_fwd_step2_uq_store", "k_fwd_small",
                     "k_fwd_small_store", "k_adj_small", "k_fwd_band", "k_fwd_band_store", "k_adj_band",
                     "k_fwd_bandk", "k_fwd_bandk_store", "k_adj_bandk"]
    assert native.tm_kernel_name(-1) is None and native.tm_kernel_name(len(names)) is None


def test_status_strings_distinct():
    s = [native.status_string(i) for i in range(7)]
    assert len(set(s)) == 7 and all(s)
    assert native.status_string(99) == "unknown status"


def test_valid_plan_and_workspace_size(wl):
    st, plan = native.tm_plan_create(make(wl), wl.cpml, wl.src, wl.rec)
    assert st == native.TM_OK and plan
    st, nbytes = native.tm_workspace_bytes(plan)
    assert st == native.TM_OK
    S, N = wl.n_shots, wl.ny * wl.nx
    snaps = 2 * wl.nt * S * (wl.pml_y1 - wl.pml_y0) * (wl.pml_x1 - wl.pml_x0) * 4
    assert snaps + 6 * S * N * 4 <= nbytes <= snaps + 6 * S * N * 4 + 16 * S * N * 4 + (1 << 20)
    native.tm_plan_destroy(plan)
    # checkpoint mode needs less memory than the full store for long runs
    long = inputs.make_config(2, n_int=40, nt=400, n_shots=2, n_rec=5)
    st, p_full = native.tm_plan_create(make(long, ckpt_every=0), long.cpml, long.src, long.rec)
    st2, p_ck = native.tm_plan_create(make(long, ckpt_every=20), long.cpml, long.src, long.rec)
    assert st == st2 == native.TM_OK
    assert native.tm_workspace_bytes(p_ck)[1] < native.tm_workspace_bytes(p_full)[1]
    bf = inputs.make_config(2, n_int=40, nt=400, n_shots=2, n_rec=5, snap="bf16")
    st3, p_bf = native.tm_plan_create(make(bf), bf.cpml, bf.src, bf.rec)
    f8 = inputs.make_config(2, n_int=40, nt=400, n_shots=2, n_rec=5, snap="fp8")
    st4, p_f8 = native.tm_plan_create(make(f8), f8.cpml, f8.src, f8.rec)
    assert st3 == st4 == native.TM_OK
    b_full, b_bf, b_f8 = (native.tm_workspace_bytes(p)[1] for p in (p_full, p_bf, p_f8))
    # snapshot store: 4, 2 and 1 byte(s) per element
    elems = 2 * 400 * 2 * 40 * 40
    assert abs((b_full - b_bf) - 2 * elems) < (1 << 20) and abs((b_bf - b_f8) - elems) < (1 << 20)
    for p in (p_full, p_ck, p_bf, p_f8):
        native.tm_plan_destroy(p)


@pytest.mark.parametrize("field,value", [
    ("order", 3), ("order", 6), ("order", 0), ("n_shots", 0), ("nt", 0), ("n_src", -1),
    ("snap", 3), ("snap", -1), ("ckpt_every", -1), ("ny", 5), ("dx", 0.0), ("dy", float("nan")),
    ("time_block", 6), ("time_block", -1), ("storage", 2), ("step_ratio", -1), ("model_per_shot", 2),
    ("model_per_shot", -1),
    ("pml_y0", 1), ("pml_x1", 10 ** 6), ("pml_y1", 20),
])
def test_invalid_descriptor(wl, field, value):
    over = {field: value}
    if field == "pml_y1":
        over["pml_y0"] = 20            # empty window
    assert create(wl, **over) == native.TM_EINVAL


def test_window_outside_grid(wl):
    p = wl.order // 2
    assert create(wl, pml_y1=wl.ny - p + 2) == native.TM_EINVAL
    assert create(wl, pml_y1=wl.ny - p + 1) == native.TM_OK      # touches the last E row


def test_invalid_indices(wl):
    p = wl.order // 2
    src = wl.src.copy()
    src[0, 0] = 1 * wl.nx + 5                     # in the zero halo (row < P)
    assert create(wl, src=src) == native.TM_EINVAL
    src[0, 0] = wl.ny * wl.nx                     # past the slab
    assert create(wl, src=src) == native.TM_EINVAL
    src[0, 0] = (wl.ny - p) * wl.nx + (wl.nx - p)  # last E cell: allowed
    assert create(wl, src=src) == native.TM_OK
    src[0, 0] = -7                                 # negative: no source
    assert create(wl, src=src) == native.TM_OK
    rec = wl.rec.copy()
    rec[1, 2] = 5 * wl.nx + (wl.nx - 1)            # last column is halo
    assert create(wl, rec=rec) == native.TM_EINVAL
    st, plan = native.tm_plan_create(make(wl), wl.cpml, None, wl.rec)
    assert st == native.TM_EINVAL                  # n_src > 0 needs indices


def test_invalid_cpml(wl):
    bad = wl.cpml.copy()
    bad[2, 0] = 0.0                                 # kappa_y = 0 on a band row
    assert create(wl, cpml=bad) == native.TM_EINVAL
    bad = wl.cpml.copy()
    bad[7, 3] = np.nan
    assert create(wl, cpml=bad) == native.TM_EINVAL
    ok = wl.cpml.copy()
    ok[2, wl.pml_y0 + 3] = 0.0                      # kappa unused off the band
    assert create(wl, cpml=ok) == native.TM_OK


def test_memory_budget(wl):
    st, plan = native.tm_plan_create(make(wl), wl.cpml, wl.src, wl.rec)
    need = native.tm_workspace_bytes(plan)[1]
    native.tm_plan_destroy(plan)
    assert create(wl, hbm_budget=need) == native.TM_OK
    assert create(wl, hbm_budget=need - 1) == native.TM_ENOMEM


def test_largest_grid_one_buffer_view():
    """A shot's state block must fit one buffer view (2^31 - 256 bytes): the
    largest square grid is accepted, one more row and column is not."""
    order, npml = 4, 8
    n = largest_square_grid(order, npml)
    for size, want in ((n, native.TM_OK), (n + 1, native.TM_EINVAL)):
        w = inputs.homogeneous_workload(order, size, size, npml, 2, (size // 2, size // 2), [(size // 2, size // 2 + 3)],
                                        seed=1)
        st, plan = native.tm_plan_create(native.make_desc(w), w.cpml, w.src, w.rec)
        if plan:
            native.tm_plan_destroy(plan)
        assert st == want, (size, st)


def test_null_arguments():
    L = native.lib()
    out = ctypes.c_void_p()
    assert L.tm_plan_create(None, None, None, None, ctypes.byref(out)) == native.TM_EINVAL
    assert L.tm_workspace_bytes(None, None) == native.TM_EINVAL
    assert L.tm_forward(None, None, 0, None, None, None, None, None, 0, 1, 0, None) == native.TM_EINVAL
    assert L.tm_adjoint(None, None, 0, None, None, None, None, None, None, None, None, None) == native.TM_EINVAL
    assert L.tm_grad(None, None, None, None, None, None) == native.TM_EINVAL
    c = ctypes.c_double(0.0)
    assert L.tm_courant_noalloc(None, None, None, None, ctypes.byref(c)) == native.TM_EINVAL


def test_call_sequence_checked_before_launch(wl):
    st, plan = native.tm_plan_create(make(wl), wl.cpml, wl.src, wl.rec)
    nbytes = native.tm_workspace_bytes(plan)[1]
    dev = FAKE_WS
    try:
        # step range
        for t0, t1 in ((0, 0), (-1, 3), (5, 4), (0, wl.nt + 1)):
            assert native.tm_forward(plan, dev, nbytes, dev, dev, dev, dev, None, t0, t1, 0, None) == native.TM_EINVAL
        # unknown flag bits
        assert native.tm_forward(plan, dev, nbytes, dev, dev, dev, dev, None, 0, 1, 8, None) == native.TM_EINVAL
        # too-small workspace / misaligned workspace
        assert native.tm_forward(plan, dev, nbytes - 1, dev, dev, dev, dev, None, 0, 1, 0, None) == native.TM_ENOMEM
        assert native.tm_forward(plan, dev + 4, nbytes, dev, dev, dev, dev, None, 0, 1, 0, None) == native.TM_EINVAL
        # missing wavelet with sources
        assert native.tm_forward(plan, dev, nbytes, dev, dev, dev, None, None, 0, 1, 0, None) == native.TM_EINVAL
        # continuing a forward that never started
        assert native.tm_forward(plan, dev, nbytes, dev, dev, dev, dev, None, 3, 5, 0, None) == native.TM_ESTATE
        # gradients without a storing forward
        assert native.tm_adjoint(plan, dev, nbytes, dev, dev, dev, dev, dev, None, dev, dev, None) == native.TM_ESTATE
        # residual required when there are receivers
        assert native.tm_adjoint(plan, dev, nbytes, dev, dev, dev, dev, None, None, None, None, None) == native.TM_EINVAL
        # shot sum needs matching pairs
        assert native.tm_grad(plan, dev, None, None, None, None) == native.TM_EINVAL
        assert native.tm_grad(plan, None, None, None, dev, None) == native.TM_EINVAL
    finally:
        native.tm_plan_destroy(plan)


def test_storage_options_exclude_checkpoints(wl):
    """Host storage and step ratios apply to the full store only."""
    assert create(wl, storage=native.TM_STORE_HOST) == native.TM_OK
    assert create(wl, step_ratio=3) == native.TM_OK
    assert create(wl, storage=native.TM_STORE_HOST, step_ratio=4) == native.TM_OK
    assert create(wl, storage=native.TM_STORE_HOST, ckpt_every=5) == native.TM_EINVAL
    assert create(wl, step_ratio=2, ckpt_every=5) == native.TM_EINVAL
    # host storage keeps only a ring of device slots in the workspace
    st, p_dev = native.tm_plan_create(make(wl), wl.cpml, wl.src, wl.rec)
    st2, p_host = native.tm_plan_create(make(wl, storage=native.TM_STORE_HOST), wl.cpml, wl.src, wl.rec)
    st3, p_r = native.tm_plan_create(make(wl, step_ratio=4), wl.cpml, wl.src, wl.rec)
    assert st == st2 == st3 == native.TM_OK
    b_dev, b_host, b_r = (native.tm_workspace_bytes(p)[1] for p in (p_dev, p_host, p_r))
    assert b_host < b_r < b_dev
    for p in (p_dev, p_host, p_r):
        native.tm_plan_destroy(p)


def test_per_shot_models_workspace(wl):
    """One model per shot keeps S model blocks [Ca | Cb | Cq] in the workspace."""
    st, p1 = native.tm_plan_create(make(wl), wl.cpml, wl.src, wl.rec)
    st2, pS = native.tm_plan_create(make(wl, model_per_shot=1), wl.cpml, wl.src, wl.rec)
    assert st == st2 == native.TM_OK
    b1, bS = native.tm_workspace_bytes(p1)[1], native.tm_workspace_bytes(pS)[1]
    slab = -(-wl.ny * wl.nx * 4 // 256) * 256
    assert bS - b1 == (wl.n_shots - 1) * 3 * slab
    native.tm_plan_destroy(p1)
    native.tm_plan_destroy(pS)
    # the Python descriptor follows the shape of the coefficient arrays
    per = inputs.per_shot_models(wl)
    assert per.ca.shape == (wl.n_shots, wl.ny, wl.nx)
    assert native.make_desc(per).model_per_shot == 1 and native.make_desc(wl).model_per_shot == 0


def test_set_indices_on_the_host(wl):
    """tm_plan_set_indices: bad indices and a geometry over the memory budget
    leave the plan unchanged; a valid one sizes the workspace like a fresh
    plan of that geometry and resets the call sequence."""
    st, plan = native.tm_plan_create(make(wl), wl.cpml, wl.src, wl.rec)
    assert st == native.TM_OK
    try:
        b0 = native.tm_workspace_bytes(plan)[1]
        assert native.lib().tm_plan_set_indices(None, None, None) == native.TM_EINVAL
        bad = wl.src.copy()
        bad[1, 0] = wl.ny * wl.nx                        # outside the grid
        assert native.tm_plan_set_indices(plan, bad, wl.rec) == native.TM_EINVAL
        bad = wl.rec.copy()
        bad[0, 1] = 0                                    # in the halo, not an E cell
        assert native.tm_plan_set_indices(plan, wl.src, bad) == native.TM_EINVAL
        assert native.tm_plan_set_indices(plan, None, wl.rec) == native.TM_EINVAL
        assert native.tm_workspace_bytes(plan)[1] == b0
        # receivers spread over many rows: more event rows, a larger workspace
        rows = wl.pml_y0 + np.arange(wl.n_rec) * 3
        rec = np.stack([rows * wl.nx + wl.pml_x0 + 2 + s for s in range(wl.n_shots)]).astype(np.int64)
        assert native.tm_plan_set_indices(plan, wl.src, rec) == native.TM_OK
        b1 = native.tm_workspace_bytes(plan)[1]
        st, fresh = native.tm_plan_create(make(wl), wl.cpml, wl.src, rec)
        assert st == native.TM_OK and native.tm_workspace_bytes(fresh)[1] == b1 > b0
        native.tm_plan_destroy(fresh)
        # the state of the old geometry is gone: gradients need a new forward
        dev = FAKE_WS
        assert native.tm_adjoint(plan, dev, b1, dev, dev, dev, dev, dev, None, dev, dev, None) == native.TM_ESTATE
        assert native.tm_forward(plan, dev, b1, dev, dev, dev, dev, None, 3, 5, 0, None) == native.TM_ESTATE
        # and back to the original geometry
        assert native.tm_plan_set_indices(plan, wl.src, wl.rec) == native.TM_OK
        assert native.tm_workspace_bytes(plan)[1] == b0
    finally:
        native.tm_plan_destroy(plan)
    # over the budget: refused, plan unchanged
    st, plan = native.tm_plan_create(make(wl, hbm_budget=b0), wl.cpml, wl.src, wl.rec)
    assert st == native.TM_OK
    try:
        assert native.tm_plan_set_indices(plan, wl.src, rec) == native.TM_ENOMEM
        assert native.tm_workspace_bytes(plan)[1] == b0
        assert native.tm_plan_set_indices(plan, wl.src, wl.rec) == native.TM_OK
    finally:
        native.tm_plan_destroy(plan)


def test_event_steps_override_is_bounded(monkeypatch):
    """TM_FDTD_EVENT_STEPS cannot push an event buffer past its size bound:
    a huge value gives the default block length (same workspace), a small
    one a smaller workspace."""
    wl = inputs.make_config(2, n_int=400, nt=30, n_shots=2, n_rec=5)    # 4 event rows of 444 cells
    st, plan = native.tm_plan_create(make(wl, nt=5000), wl.cpml, wl.src, wl.rec)
    b_default = native.tm_workspace_bytes(plan)[1]
    native.tm_plan_destroy(plan)
    monkeypatch.setenv("TM_FDTD_EVENT_STEPS", str(1 << 40))
    st, plan = native.tm_plan_create(make(wl, nt=5000), wl.cpml, wl.src, wl.rec)
    assert st == native.TM_OK
    # (the default rounds the block down to an even length: at most one
    # step of the four event buffers apart; unbounded, 5000 steps would
    # add about 33 MB)
    one_step = 4 * 4 * wl.nx * 4
    assert abs(native.tm_workspace_bytes(plan)[1] - b_default) <= one_step + 4 * 256
    native.tm_plan_destroy(plan)
    monkeypatch.setenv("TM_FDTD_EVENT_STEPS", "8")
    st, plan = native.tm_plan_create(make(wl, nt=5000), wl.cpml, wl.src, wl.rec)
    assert st == native.TM_OK
    assert native.tm_workspace_bytes(plan)[1] < b_default
    native.tm_plan_destroy(plan)
