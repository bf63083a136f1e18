"""The benchmark's byte model (bench.kernel_bytes) on the CPU: every kernel
the library times has one, and the figures follow the per-cell accounting
written out in the function's docstring (so that a renamed kernel or a
changed formula cannot silently drop out of the roofline line)."""

import os
import sys

import pytest

from tm_maxwell_fdtd_amd import inputs, native

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


@pytest.fixture(scope="module")
def wl():
    return inputs.as_f32(inputs.random_workload(4, 40, 7, nt=30, n_shots=3, n_src=2, n_rec=4, seed=1500))


def test_every_timed_kernel_has_a_byte_model(wl):
    names = [native.tm_kernel_name(k) for k in range(native.tm_kernel_count())]
    for name in names:
        b = bench.kernel_bytes(name, wl, bench.stores(name), 4)
        assert b is not None and b > 0, name


def test_one_step_counts(wl):
    p = wl.order // 2
    S = wl.n_shots
    cells = (wl.ny - 2 * p) * (wl.nx - 2 * p)
    nyi, nxi = wl.pml_y1 - wl.pml_y0, wl.pml_x1 - wl.pml_x0
    interior = nyi * nxi
    ny_e, nx_e = wl.ny - 2 * p, wl.nx - 2 * p
    band = (ny_e - (nyi - 1)) * nx_e + (nx_e - (nxi - 1)) * ny_e
    fwd = S * (36 * cells + 16 * band)
    assert bench.kernel_bytes("k_fwd_step", wl, False, 4) == fwd
    assert bench.kernel_bytes("k_fwd_step_store", wl, False, 4) == fwd + S * 8 * interior
    assert bench.kernel_bytes("k_fwd_step_store", wl, False, 2) == fwd + S * 4 * interior
    assert bench.kernel_bytes("k_fwd_step2", wl, False, 4) == 2 * fwd
    assert bench.kernel_bytes("k_fwd_step2_uq", wl, False, 4) == 2 * S * (32 * cells + 16 * band)
    adj = S * (36 * cells + 16 * band)
    assert bench.kernel_bytes("k_adj_step", wl, False, 4) == adj
    assert bench.kernel_bytes("k_adj_step", wl, True, 4) == adj + S * (8 + 16) * interior
    assert bench.kernel_bytes("k_adj_step2_uq", wl, True, 2) == 2 * S * (32 * cells + 16 * band + 20 * interior)


def test_resident_counts(wl):
    p = wl.order // 2
    S = wl.n_shots
    full = wl.ny * wl.nx
    nyi, nxi = wl.pml_y1 - wl.pml_y0, wl.pml_x1 - wl.pml_x0
    interior = nyi * nxi
    ny_e, nx_e = wl.ny - 2 * p, wl.nx - 2 * p
    band = (ny_e - (nyi - 1)) * nx_e + (nx_e - (nxi - 1)) * ny_e
    base = S * (8 * (3 * full + 2 * band) + 12 * full)
    for name in ("k_fwd_small", "k_fwd_band", "k_fwd_bandk"):
        assert bench.kernel_bytes(name, wl, False, 4) == base
        assert bench.kernel_bytes(name + "_store", wl, False, 4, run_steps=10) == base + S * 10 * 8 * interior
    for name in ("k_adj_small", "k_adj_band", "k_adj_bandk"):
        assert bench.kernel_bytes(name, wl, True, 4, run_steps=10) == base + S * (10 * 8 + 16) * interior
