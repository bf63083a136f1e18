#!/usr/bin/env python3
"""Throughput of the TM FDTD hot path on one MI355X.

One step = one pass of the whole path over one batch of shots: tm_forward
with storage (stencil steps, source injection, receiver gather, snapshot
epilogue), tm_adjoint (residual injection, exact adjoint steps, gradient
accumulation; segment replay in checkpoint mode) and tm_grad (shot sum), on
the order-8 workload: 1024x1024 interior + 32-cell CPML per side, 16 shots,
2000 time steps, bfloat16 snapshots.  The misfit is J = 1/2 |r|^2, so the
adjoint source is the records themselves.

tm_forward is called with TM_FWD_CHECK (Courant check, which also finds
whether Cq holds one value: mu_r = 1 in these workloads, so the forward
kernels read no Cq array), inside the timed region.

value = cell-updates / time of one step (Gcell-updates/s), where
cell-updates = shots x (interior + CPML cells) x time steps.  The forward
pass alone (no storage) is timed as well and reported as ``fwd_value``.

The ``roofline`` object is for the dominant stencil kernel: algorithmic
bytes per launch over its average launch duration, sampled with HIP events
inside the library on the stream the kernels run on (tm_timing_*).  HBM
traffic comes from rocprofv3 FETCH_SIZE / WRITE_SIZE counters recorded in
``profiles/`` (bytes per launch, scaled by what the counters read for a
plain 1 GiB copy), is reported as a rate over the same launch time as
``achieved`` and is used only while the kernel source is unchanged.

``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload (one shot, a few dozen time steps) on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Gcell-updates/s fwd and fwd+adjoint (8th order) + % of HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
WORKLOADS = {
    3: "order-8 TM FDTD, 1024x1024 interior + 32-cell CPML (1096x1096 padded), 16 shots, "
       "2000 steps, 256 receivers/shot, 600 MHz Ricker, bf16 snapshots, fwd(store)+adjoint+shot-sum",
    2: "order-4 TM FDTD, 256x256 interior + 20-cell CPML, 4 shots, 1000 steps, fp32 snapshots",
    5: "order-4 TM FDTD, 384x384 interior + 20-cell CPML, 128 shots, 800 steps, fp32 snapshots",
    4: "order-8 TM FDTD, 4096x4096 interior + 40-cell CPML, 8 shots, 4000 steps, fp32, "
       "checkpoint every 64 steps + segment replay",
    1: "order-2 TM FDTD, 64x64 interior + 10-cell CPML, 1 shot, 300 steps, fp32 snapshots",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic bytes per launch of each stencil kernel.  Per cell of the
# launch: every field and coefficient the update reads once, every field it
# writes once, the CPML memory read-modify-write on band cells, the snapshot
# writes / reads and the gradient read-modify-write on interior cells.
# ---------------------------------------------------------------------------

def _counts(wl):
    p = wl.order // 2
    cells = (wl.ny - 2 * p) * (wl.nx - 2 * p)                  # per shot
    nyi, nxi = wl.pml_y1 - wl.pml_y0, wl.pml_x1 - wl.pml_x0
    interior = nyi * nxi
    ny_e, nx_e = wl.ny - 2 * p, wl.nx - 2 * p
    yband_rows = ny_e - (nyi - 1)                               # H flag: outside [y0, y1-1)
    xband_cols = nx_e - (nxi - 1)
    band_y = yband_rows * nx_e                                  # cells in y bands
    band_x = xband_cols * ny_e
    return cells, interior, band_y, band_x


def kernel_bytes(name, wl, store, snap_bytes, run_steps=None):
    """Algorithmic HBM bytes of one launch of kernel ``name`` (all shots).

    k_fwd_step: read E, Hx, Hz, Ca, Cb, Cq and write E, Hx, Hz (36 B per
    cell); read-modify-write of one H-update and one E-update CPML memory
    per band axis (16 B per band cell and axis); with storage, Ey^n and
    curl H^n of every interior cell (2 x 4 B, or 2 x 2 B in bf16).
    k_adj_step: the same 36 B for the adjoint fields and coefficients, the
    same 16 B per band cell and axis for the four adjoint memories, and on
    interior cells the two snapshot reads plus the read-modify-write of the
    two per-shot gradients (16 B).
    k_fwd_step2 / k_adj_step2 advance two time steps per launch: twice the
    bytes of k_fwd_step / k_adj_step (the per-cell-update figure times the
    cell-updates of the launch), although the state crosses HBM only once.
    k_fwd_step2_uq / k_adj_step2_uq are the instances where Cq holds one
    value and is not read: 32 B per cell instead of 36.  A "_store" suffix
    names the forward launches that store snapshots (the library times them
    apart); ``stores(name)`` gives ``store`` for a timed name.
    """
    if name.endswith("_store"):
        name, store = name[:-len("_store")], True
    cells, interior, band_y, band_x = _counts(wl)
    S = wl.n_shots
    if name in ("k_fwd_small", "k_adj_small", "k_fwd_band", "k_adj_band", "k_fwd_bandk", "k_adj_bandk"):
        # resident kernels: one launch runs a whole event block (run_steps
        # steps, the whole run if not given) on chip; HBM sees the state in
        # and out (fields and band memories), the model once, and per step
        # the snapshots (and in the adjoint the gradients once, read and
        # written)
        p = wl.order // 2
        full = wl.ny * wl.nx
        state = 2 * 4 * (3 * full + 2 * (band_y + band_x))
        steps = wl.nt if run_steps is None else run_steps
        snaps = steps * 2 * snap_bytes * interior if store else 0
        grads = 16 * interior if (store and name.startswith("k_adj")) else 0
        return S * (state + 12 * full + snaps + grads)
    if name in ("k_fwd_step", "k_fwd_step_uq"):
        snaps = 2 * snap_bytes * interior if store else 0
        per_cell = 32 if name.endswith("_uq") else 36
        return S * (per_cell * cells + 16 * (band_y + band_x) + snaps)
    if name == "k_fwd_step2":
        return 2 * kernel_bytes("k_fwd_step", wl, store, snap_bytes)
    if name == "k_fwd_step2_uq":
        return 2 * kernel_bytes("k_fwd_step_uq", wl, store, snap_bytes)
    if name in ("k_adj_step", "k_adj_step_uq"):
        grads = (2 * snap_bytes + 16) * interior if store else 0
        per_cell = 32 if name.endswith("_uq") else 36
        return S * (per_cell * cells + 16 * (band_y + band_x) + grads)
    if name == "k_adj_step2":
        return 2 * kernel_bytes("k_adj_step", wl, store, snap_bytes)
    if name == "k_adj_step2_uq":
        return 2 * kernel_bytes("k_adj_step_uq", wl, store, snap_bytes)
    return None


def stores(name):
    """Whether launches timed under ``name`` store snapshots (forward) or
    accumulate gradients (adjoint) in a full forward + adjoint step."""
    return name.endswith("_store") or name.startswith("k_adj")


def kernel_source_sha():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tm_maxwell_fdtd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".h")):
            with open(os.path.join(csrc, name), "rb") as fh:
                h.update(name.encode())
                h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, cfg):
    """Measured HBM bytes per launch, if recorded for the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_config{cfg}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_src_sha") != kernel_source_sha():
        return None
    return float(rec["hbm_bytes_per_launch"])


# ---------------------------------------------------------------------------

def cpu_info():
    """CPU model, physical cores and the CPUs this process may run on."""
    model, cores = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                elif not key and phys is not None and core is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count()
    return {"cpu_model": model, "physical_cores": len(cores) or None, "logical_cpus": os.cpu_count(),
            "cpus_available": avail}


def cpu_baseline(wl, steps, min_seconds=10.0, max_runs=24):
    """fp64 oracle on one shot of the workload for ``steps`` time steps.

    The sample (forward with storage, then the exact adjoint) is repeated
    until at least ``min_seconds`` of CPU work has been timed; the rate is
    total cell-updates over total time.  The forward alone (no storage) is
    timed the same way for ``fwd_value``.
    """
    import dataclasses

    import oracle

    one = dataclasses.replace(wl, n_shots=1, nt=steps, src=wl.src[:1].copy(), rec=wl.rec[:1].copy(),
                              f=wl.f[:steps, :1].copy())
    p = wl.order // 2
    cells = (wl.ny - 2 * p) * (wl.nx - 2 * p) * steps

    def rate(fn):
        total, runs = 0.0, 0
        while runs < max_runs and (runs == 0 or total < min_seconds):
            t0 = time.perf_counter()
            fn()
            total += time.perf_counter() - t0
            runs += 1
        return cells * runs / total / 1e9, runs, total

    def fwd_adj():
        r, _, snaps = oracle.forward(one, store=True)
        oracle.adjoint(one, r, snaps)

    value, runs, total = rate(fwd_adj)
    fwd_value, fruns, ftotal = rate(lambda: oracle.forward(one))
    out = {"value": value, "unit": "Gcell-updates/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"1 of {wl.n_shots} shots, {steps} of {wl.nt} time steps, same grid and model; "
                     f"forward with storage + exact adjoint in fp64, {runs} run(s), {total:.1f} s; "
                     f"forward alone {fruns} run(s), {ftotal:.1f} s",
           "fwd_value": fwd_value, "threads": oracle.num_threads()}
    out.update(cpu_info())
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=3, choices=sorted(WORKLOADS))
    ap.add_argument("--timing-every", type=int, default=0,
                    help="sample the stencil launches starting at every k-th time step with HIP events "
                         "(0: 8, and 1 for configs 1 and 2, whose resident kernels run a block of "
                         "steps per launch)")
    ap.add_argument("--cpu-steps", type=int, default=200, help="time steps of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fwd", action="store_true", help="skip the forward-only timing")
    ap.add_argument("--nt", type=int, default=0,
                    help="override the number of time steps (profiling runs only; "
                         "the bench line then names the reduced workload)")
    ap.add_argument("--time-block", type=int, default=0, choices=(0, 1, 2, 3, 4, 5),
                    help="time steps per launch of the forward and the adjoint (0: the default, 2)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel for calibrating HBM byte counters)")
    args = ap.parse_args()
    if args.timing_every <= 0:
        args.timing_every = 1 if args.config in (1, 2) else 8

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(shots would be sharded across GPUs with one gradient all-reduce; not built).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from tm_maxwell_fdtd_amd import inputs, native

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    native.lib()                 # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_mb > 0:
        n = args.copy_mb * (1 << 20) // 4
        src_t = torch.ones(n, dtype=torch.float32, device=dev)
        dst_t = torch.empty_like(src_t)
        torch.cuda.synchronize()
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.copy_mb} MiB done")
        del src_t, dst_t

    log(f"building workload config{args.config}")
    over = {"nt": args.nt} if args.nt > 0 else {}
    wl = inputs.as_f32(inputs.make_config(args.config, **over))
    prop = native.Propagator(wl, device=dev, time_block=args.time_block)
    log(f"workspace {prop.ws_bytes / 2**30:.1f} GiB, grid {wl.ny}x{wl.nx}, S={wl.n_shots}, nt={wl.nt}")
    S, ny, nx = wl.n_shots, wl.ny, wl.nx
    f32 = dict(dtype=torch.float32, device=dev)
    r = torch.zeros((wl.nt, S, wl.n_rec), **f32)
    grad_f = torch.empty((wl.nt, S, wl.n_src), **f32)
    gca_s = torch.empty((S, ny, nx), **f32)
    gcb_s = torch.empty((S, ny, nx), **f32)
    gca = torch.empty((ny, nx), **f32)
    gcb = torch.empty((ny, nx), **f32)
    P = native.ptr
    ws, wsb = P(prop.ws), prop.ws_bytes
    ca, cb, cq, f = P(prop.ca), P(prop.cb), P(prop.cq), P(prop.f)
    courant = prop.courant()
    log(f"Courant number {courant:.4f}")

    def stream():
        return native.stream_handle()

    def step():
        st = native.tm_forward(prop.plan, ws, wsb, ca, cb, cq, f, P(r), 0, wl.nt,
                               native.TM_FWD_STORE | native.TM_FWD_CHECK, stream())
        assert st == 0, native.status_string(st)
        # J = 1/2 |r|^2: dJ/dr = r
        st = native.tm_adjoint(prop.plan, ws, wsb, ca, cb, cq, f, P(r), P(grad_f), P(gca_s), P(gcb_s), stream())
        assert st == 0, native.status_string(st)
        st = native.tm_grad(prop.plan, P(gca_s), P(gcb_s), P(gca), P(gcb), stream())
        assert st == 0, native.status_string(st)

    def fwd_only():
        st = native.tm_forward(prop.plan, ws, wsb, ca, cb, cq, f, P(r), 0, wl.nt, native.TM_FWD_CHECK, stream())
        assert st == 0, native.status_string(st)

    cell_updates = wl.cell_updates()

    def timed(fn, k, w, label):
        for i in range(w):
            fn()
            torch.cuda.synchronize()
            log(f"{label} warmup {i + 1}/{w} done")
        native.tm_timing_read(prop.plan)                      # discard warmup samples
        native.tm_timing_enable(prop.plan, args.timing_every)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for i in range(k):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        native.tm_timing_enable(prop.plan, 0)
        st, kt = native.tm_timing_read(prop.plan)
        assert st == 0
        ev_ms = e0.elapsed_time(e1)
        log(f"{label}: {k} steps, wall {wall:.3f} s, events {ev_ms / 1e3:.3f} s")
        return wall, ev_ms / 1e3, kt

    results = {}
    if not args.no_fwd:
        wall, ev, kt = timed(fwd_only, args.steps, args.warmup, "forward")
        results["fwd"] = (max(wall, ev), kt)
    wall, ev, kt = timed(step, args.steps, args.warmup, "fwd+adj")
    results["step"] = (max(wall, ev), kt)
    ok = bool(torch.isfinite(gca).all() and torch.isfinite(gcb).all() and torch.isfinite(r).all())
    if not ok:
        log("non-finite values in the outputs")

    t_step = results["step"][0] / args.steps
    value = cell_updates / t_step / 1e9
    fwd_value = cell_updates / (results["fwd"][0] / args.steps) / 1e9 if "fwd" in results else None

    # roofline of the dominant kernel of the full step
    snap_bytes = 2 if wl.snap == "bf16" else 4
    kernels = {}
    for name, (ms, n) in results["step"][1].items():
        if n == 0:
            continue
        avg_ms = ms / n
        # launches of the sampled steps: every timing_every-th step's launch
        # (a two-step launch covers two steps)
        per_launch = 2 if name.startswith(("k_fwd_step2", "k_adj_step2")) else 1
        launches = n * args.timing_every / per_launch / args.steps
        # resident kernels: one launch per event block, all sampled at
        # timing_every 1; their steps per launch from the launch count
        resident = name.startswith(("k_fwd_small", "k_adj_small", "k_fwd_band", "k_adj_band"))
        if resident:
            launches = n / args.steps if args.timing_every == 1 else launches
        run_steps = wl.nt / launches if resident and launches > 0 else None
        # the adjoint accumulates gradients on every launch of a full step
        nbytes = kernel_bytes(name, wl, store=stores(name), snap_bytes=snap_bytes, run_steps=run_steps)
        kernels[name] = dict(avg_us=avg_ms * 1e3, samples=n, est_total_s=avg_ms * launches / 1e3,
                             alg_bytes=nbytes, gbs=nbytes / (avg_ms * 1e-3) / 1e9)
    dom = max(kernels, key=lambda k: kernels[k]["est_total_s"])
    kd = kernels[dom]
    # measured HBM bytes per launch (counter run of the same kernel source), as
    # a rate over the same average launch time as ``achieved``
    traffic_b = load_traffic(dom, args.config)
    traffic = None if traffic_b is None else round(traffic_b / (kd["avg_us"] * 1e-6) / 1e9, 1)
    roofline = {"bound": "hbm", "achieved": round(kd["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kd["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_frac": None if traffic is None else round(traffic / HBM_PEAK_GBS, 4),
                "kernel": dom, "avg_launch_us": round(kd["avg_us"], 2), "alg_bytes_per_launch": kd["alg_bytes"],
                "traffic_bytes_per_launch": None if traffic_b is None else int(traffic_b)}
    for name, k in sorted(kernels.items()):
        log(f"  {name:20s} avg {k['avg_us']:9.2f} us  ({k['samples']} samples)  "
            f"alg {k['alg_bytes'] / 1e6:8.1f} MB  -> {k['gbs']:7.1f} GB/s  est {k['est_total_s']:.3f} s/step")
    fwd_kern = {}
    if "fwd" in results:
        for name, (ms, n) in results["fwd"][1].items():
            if n:
                rs = None
                if name.startswith(("k_fwd_small", "k_fwd_band")) and args.timing_every == 1:
                    rs = wl.nt / (n / args.steps)
                nb = kernel_bytes(name, wl, store=stores(name), snap_bytes=snap_bytes, run_steps=rs)
                fwd_kern[name] = dict(avg_us=round(ms / n * 1e3, 2),
                                      gbs=round(nb / (ms / n * 1e-3) / 1e9, 1))

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "Gcell-updates/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"config{args.config}: " + WORKLOADS[args.config]
                   + (f" (reduced to {wl.nt} time steps)" if args.nt > 0 else ""),
                   "grid": [wl.ny, wl.nx], "shots": wl.n_shots, "time_steps": wl.nt, "order": wl.order,
                   "snapshots": wl.snap, "ckpt_every": wl.ckpt_every, "cell_updates": cell_updates},
        "fwd_value": None if fwd_value is None else round(fwd_value, 3),
        "fwd_kernels": fwd_kern,
        "roofline": roofline,
        "outputs_finite": ok,
    }
    prop.close()
    del prop
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log(f"timing the fp64 oracle on {args.cpu_steps} steps of one shot")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_steps)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
