/*
 * tm_fdtd.h -- C ABI of the MI355X (gfx950) 2-D TM Maxwell FDTD propagator
 * with its exact discrete adjoint and the model gradients dJ/dCa, dJ/dCb.
 *
 * Source of the method: tide-GPR 0.0.9, tide/csrc/maxwell.cu (the header
 * comment's discrete equations, the kernels forward_kernel_h/_e, the
 * storing variants, add_sources_ey, record_receivers_ey,
 * add_adjoint_sources_ey, record_adjoint_at_sources, combine_grad and the
 * host launchers forward, forward_with_storage and backward).
 *
 * Grid and index conventions (all per shot, row-major, x fastest):
 *   ny x nx padded grid, P = order / 2, flat cell index y * nx + x.
 *   Ey is updated on P <= y <= ny-P, P <= x <= nx-P;
 *   Hx on P <= y <= ny-P-1, P <= x <= nx-P (the point y + 1/2 stored at y);
 *   Hz on P <= y <= ny-P,   P <= x <= nx-P-1 (the point x + 1/2 stored at x).
 *   The interior window [pml_y0, pml_y1) x [pml_x0, pml_x1) is the region
 *   without CPML; E derivatives are CPML-filtered outside it, H derivatives
 *   outside [pml_y0, pml_y1 - 1) (resp. x), as in the page's kernels.
 *   Gradients are accumulated on the interior window only.
 *
 * One step n (forward_kernel_h, forward_kernel_e, add_sources_ey,
 * record_receivers_ey, in that order):
 *   Hx -= Cq * filt(Dz^h Ey);  Hz += Cq * filt(Dx^h Ey)
 *   Ey  = Ca * Ey + Cb * (filt(Dx Hz) - filt(Dz Hx))
 *   Ey[src] += f[n];  r[n] = Ey[rec]
 * with filt(d) = d / kappa + m, m <- b m + a d on the CPML bands.
 *
 * Memory ownership: every array argument of tm_forward, tm_adjoint,
 * tm_grad and tm_courant is a device pointer owned by the caller.  The
 * workspace is caller-allocated device memory of at least
 * tm_workspace_bytes() bytes; it holds the wavefields, the band-only CPML
 * memories, the snapshot store (or checkpoints and a replay segment) and
 * small tables.  A plan owns host memory only.  Every call is asynchronous
 * on ``stream`` (a hipStream_t; NULL = the null stream) unless stated.
 * A plan also holds the state of a forward/adjoint sequence (the step the
 * forward reached, which workspace it used, what its checks found), so
 * calls on one plan must not run concurrently from several host threads;
 * separate plans are independent.
 *
 * Errors: argument errors are detected on the host before any launch and
 * returned as a tm_status; nothing is printed and nothing aborts.
 */
#ifndef TM_FDTD_H
#define TM_FDTD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tm_status {
    TM_OK = 0,
    TM_EINVAL = 1,      /* invalid descriptor, pointer, size or index          */
    TM_EUNSTABLE = 2,   /* Courant number of the model above 1                 */
    TM_ENOMEM = 3,      /* workspace too small, or plan over the HBM budget    */
    TM_EHIP = 4,        /* a HIP runtime call or kernel launch failed          */
    TM_ESTATE = 5,      /* call sequence: e.g. adjoint without a storing forward */
    TM_ENONFINITE = 6   /* non-finite value detected                           */
} tm_status;

typedef enum tm_snap {
    TM_SNAP_F32 = 0,    /* snapshots stored as float32                          */
    TM_SNAP_BF16 = 1,   /* snapshots stored as bfloat16, round-to-nearest-even  */
    TM_SNAP_FP8 = 2     /* snapshots stored as OCP FP8 E4M3 (E4M3FN: bias 7, no
                           infinities, max 448), round-to-nearest-even, finite
                           values saturated at +-448 (tm_fp8_encode)          */
} tm_snap;

/* tm_forward flags */
#define TM_FWD_STORE 1  /* keep what tm_adjoint needs: snapshots, or checkpoints */
#define TM_FWD_CHECK 2  /* check the Courant number before stepping (synchronises) */

typedef enum tm_storage {
    TM_STORE_DEVICE = 0,    /* snapshots in the device workspace                */
    TM_STORE_HOST = 1       /* snapshots in a pinned host store that the plan
                               allocates at the first storing forward (size
                               ceil(nt / step_ratio) * 2 * S * ny_i * nx_i *
                               element bytes); the workspace holds a ring of 3
                               device slots, copied out after each stored step
                               on a copy stream of the plan and prefetched back
                               in the adjoint.  Not with checkpoints.          */
} tm_storage;

typedef struct tm_desc {
    int32_t order;          /* spatial order: 2, 4 or 8                         */
    int32_t snap;           /* tm_snap                                          */
    int64_t n_shots;        /* shots S (sharing one model unless model_per_shot) */
    int64_t ny, nx;         /* padded grid; ny * nx < 2^29                      */
    int64_t pml_y0, pml_y1; /* interior window rows [pml_y0, pml_y1)            */
    int64_t pml_x0, pml_x1; /* interior window columns [pml_x0, pml_x1)         */
    double dy, dx;          /* grid spacing in metres (kernels use 1/dy, 1/dx)  */
    int64_t nt;             /* time steps                                       */
    int64_t n_src, n_rec;   /* sources and receivers per shot (may be 0)        */
    int64_t ckpt_every;     /* 0: store every step; K > 0: checkpoint the state
                               every K steps and replay segments in tm_adjoint  */
    uint64_t hbm_budget;    /* bytes the workspace may use; 0 = unlimited       */
    int32_t time_block;     /* how the steps are launched: 1 = one step per
                               launch of the streaming kernels; 2 = two steps
                               in one pass over the state (the adjoint pairs
                               steps only with the snapshots in device
                               memory); 3 = resident kernels wherever the grid
                               fits one workgroup's LDS (ny * nx < 8192, a
                               whole run of steps per launch, one workgroup
                               per shot; snapshots in device memory and no
                               checkpoints, else 2); 4 = banded resident
                               kernels wherever they fit (each shot in bands
                               of rows, one workgroup per band, a whole run
                               of steps per launch, neighbouring bands
                               exchanging halo rows every step; ny < 2048,
                               every band's workgroup resident at once, same
                               conditions as 3, else 2); 5 = as 4, with
                               blocked banded kernels where they fit (every
                               band also steps the 3(2P-1) rows next to it
                               on each side, else 2(2P-1), at most 2048
                               cells in all, so that neighbouring bands
                               exchange their whole state only every third,
                               else every second, step), else as 4;
                               0 = default: 3 with 16
                               shots or more, else, where the streaming
                               kernels would leave most of the device idle,
                               5 at order 2 and 4 at orders 4 and 8, else 2.
                               All give bitwise the same results.
                               A banded launch whose exchange wait fails
                               makes the call return TM_EHIP (never
                               expected; its outputs are then undefined;
                               not detected in calls captured in a HIP
                               graph, which the calls otherwise support).    */
    int32_t storage;        /* tm_storage: where a storing forward keeps the
                               snapshots (full-store mode only)                */
    int64_t step_ratio;     /* store snapshots (and accumulate gradients) every
                               step_ratio-th step only, weighting each term by
                               step_ratio (an approximation); 0 or 1 = every
                               step.  Full-store mode only.                     */
    int32_t model_per_shot; /* 0: one model for all shots, the coefficient
                               arrays are [ny][nx]; 1: one model per shot
                               (batched models), [S][ny][nx], and each shot's
                               gradient belongs to its own model              */
    int32_t reserved;       /* 0                                                */
} tm_desc;

typedef struct tm_plan tm_plan;

/*
 * Validate a problem and build a plan (host only, no HIP call).
 * Defined by: the set-up part of the page's host launchers forward,
 * forward_with_storage and backward (grid sizes, 1/dy and 1/dx, the CPML
 * window pml_y0..pml_x1, sources and receivers per shot, shot-batched or
 * shared models), which this plan does once instead of per call.
 * Why the source and receiver cells are plan arguments and not per-call
 * ones (the page's launchers take them per call): the step kernels inject
 * and record through host-built per-row tables (event rows: the grid rows
 * holding sources or receivers, the distinct cells on them, CSR lists of
 * the entries of each cell), whose size sets part of the workspace layout.
 * A new acquisition geometry on the same grid is set with
 * tm_plan_set_indices, without a new plan.
 *   cpml: host float32 [12][max(ny, nx)]: ay, by, ky, ayh, byh, kyh (first
 *         ny entries used) then ax, bx, kx, axh, bxh, kxh (first nx used);
 *         the integer-grid arrays filter E-update derivatives, the half-grid
 *         ones H-update derivatives.  kappa must be nonzero on the bands.
 *   src:  host int64 [S][n_src] flat cell indices y*nx+x (may be NULL when
 *         n_src == 0); rec: host int64 [S][n_rec].  A negative index means
 *         "no source/receiver"; any other index must be an Ey cell.  Several
 *         sources (receivers) of one shot may share a cell: they add up.
 * Returns TM_EINVAL on an inconsistent descriptor (order not in {2,4,8},
 * grid too small, window outside [P, n-P], empty window, ny*nx >= 2^29,
 * one shot's state block (Ey, Hx, Hz and the band memories, about
 * 12 ny nx bytes; 13363 x 13363 at order 4 with 8-cell bands is the
 * largest square grid) over 2^31 - 256 bytes, bad indices,
 * ckpt_every < 0), TM_ENOMEM when the workspace would exceed hbm_budget.
 * The plan copies everything it needs.
 */
tm_status tm_plan_create(const tm_desc* desc, const float* cpml, const int64_t* src,
                         const int64_t* rec, tm_plan** out);

/* Frees the plan and the host memory it allocated (pinned staging and
 * read-back buffers, the pinned snapshot store of TM_STORE_HOST), after
 * waiting for the work that uses it. */
void tm_plan_destroy(tm_plan* plan);

/*
 * Replace the plan's source and receiver cells (a new acquisition geometry
 * with the same n_src and n_rec per shot; same conventions as
 * tm_plan_create: host int64 [S][n_src] and [S][n_rec], negative = none).
 * Defined by: the src / rec index arguments of the page's launchers
 * (forward, forward_with_storage, backward) and the kernels that use them
 * (add_sources_ey, record_receivers_ey, add_adjoint_sources_ey,
 * record_adjoint_at_sources).
 * The event-row tables are rebuilt, so the workspace size may change:
 * query tm_workspace_bytes again (a smaller workspace than it reports is
 * rejected with TM_ENOMEM by the device calls).  The sequence state is
 * reset: tm_adjoint needs a new storing tm_forward (else TM_ESTATE).  When
 * the plan has run on a device, the call waits for that device
 * (hipDeviceSynchronize) before it frees the plan's pinned staging copy of
 * the old tables.  Errors (TM_EINVAL: a bad index; TM_ENOMEM: over
 * hbm_budget; TM_EHIP: the wait failed) leave the plan unchanged.
 */
tm_status tm_plan_set_indices(tm_plan* plan, const int64_t* src, const int64_t* rec);

/* Bytes of device workspace the plan needs (host only). */
tm_status tm_workspace_bytes(const tm_plan* plan, uint64_t* bytes);

/*
 * Courant number sqrt(max(Cb*Cq)) * sum|c_k| * sqrt(1/dx^2 + 1/dy^2) of a
 * model (the stability limit of the staggered leapfrog scheme; the page
 * gives none, its launchers do not check stability) (the largest over the shots' models with model_per_shot); the
 * scheme is stable when it is at most 1.  cb, cq: device float32 [ny][nx]
 * ([S][ny][nx] with model_per_shot).  Uses the workspace's scratch area and
 * synchronises ``stream`` (the result comes back through a few KiB of
 * pinned host memory that the plan allocates at its first read-back and
 * tm_plan_destroy frees; tm_forward's check and the banded kernels' failure
 * word use them too).
 */
tm_status tm_courant(tm_plan* plan, void* ws, uint64_t ws_bytes, const float* cb,
                     const float* cq, void* stream, double* courant);

/*
 * tm_courant without a workspace, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation) or that check a model before allocating the workspace.
 * Same result as tm_courant (bitwise; same kernel).  Its scratch (513
 * floats: 256 per-block maxima, 256 per-block flags of the uniform-Cq test
 * and cq[0]) is a static device array of the library, one per device, held
 * until the process ends; the scratch size does not depend on the model
 * size, so no size is refused for it.  Allocates nothing (no hipMalloc /
 * hipFree, no pinned host memory: the result is read back into memory of
 * the call), synchronises ``stream``.  Calls that overlap on one device share the
 * array and race: serialise them.  TM_EINVAL for a NULL argument or a
 * device ordinal of 64 or more; TM_EHIP when the array's device address
 * cannot be found.
 */
tm_status tm_courant_noalloc(tm_plan* plan, const float* cb, const float* cq, void* stream,
                             double* courant);

/*
 * Forward propagation of all shots over steps [t0, t1), 0 <= t0 < t1 <= nt.
 * Defined by: the page's host launchers forward (without TM_FWD_STORE) and
 * forward_with_storage (with it), and the per-step order of their loop:
 * forward_kernel_h, forward_kernel_e / forward_kernel_e_with_storage(_bf16,
 * _fp8), add_sources_ey, record_receivers_ey; the header comment's forward
 * equations.  The launchers' start_t / nt chunking is t0 / t1 here.
 * t0 == 0 starts from zero fields; t0 > 0 continues the state a previous
 * call on the same workspace left at step t0 (else TM_ESTATE).
 *   ca, cb, cq: device float32 [ny][nx] update coefficients ([S][ny][nx],
 *      shot s's model at s, with model_per_shot).
 *   f: device float32 [nt][S][n_src] source amplitudes, added to Ey after
 *      the E update of step n (required when n_src > 0).
 *   r: device float32 [nt][S][n_rec]; rows t0..t1-1 receive Ey at the
 *      receivers after the injection of the same step (0 for a negative
 *      index).  May be NULL.
 *   flags: TM_FWD_STORE keeps what tm_adjoint needs (every chunk from
 *      t0 = 0 to nt must pass it); TM_FWD_CHECK returns TM_EUNSTABLE before
 *      stepping when the Courant number exceeds 1.  The same check finds
 *      whether every value of cq (all shots' models) has the bits of cq[0]
 *      (mu_r uniform); the call then runs forward kernels that use that
 *      value instead of reading the array, with bitwise the same results.
 */
tm_status tm_forward(tm_plan* plan, void* ws, uint64_t ws_bytes, const float* ca,
                     const float* cb, const float* cq, const float* f, float* r,
                     int64_t t0, int64_t t1, int32_t flags, void* stream);

/*
 * Exact discrete adjoint (time-reversed transpose of the forward step, CPML
 * included) over all nt steps, after a storing tm_forward that reached nt on
 * the same workspace (else TM_ESTATE).  May be called repeatedly.
 * Defined by: the page's host launcher backward (its reverse time loop:
 * add_adjoint_sources_ey, record_adjoint_at_sources, backward_kernel_lambda_h,
 * backward_kernel_lambda_e_with_grad) and the header comment's adjoint
 * equations (the forward run backwards in time with transposed operators)
 * and gradients (dJ/dCa = sum_n lambda^{n+1} Ey^n, dJ/dCb = sum_n
 * lambda^{n+1} curlH^n).  Unlike the page's kernels, the transpose here is
 * exact for heterogeneous Cb, Cq and inside the CPML bands (the coefficient
 * at the source point, then that point's filter run backwards in time,
 * then the transposed stencil).
 *   ca, cb, cq, f: the same arrays as the forward (f is re-read by the
 *      segment replay of checkpoint mode; when the forward's TM_FWD_CHECK
 *      found cq to hold one value and cq is the same pointer, the adjoint
 *      steps and the replays use that value instead of reading the array,
 *      with bitwise the same results).
 *   grad_r: device float32 [nt][S][n_rec], dJ/dr (required when n_rec > 0).
 *   grad_f: device float32 [nt][S][n_src], receives dJ/df (adjoint field at
 *      the sources); may be NULL.
 *   grad_ca_shot, grad_cb_shot: device float32 [S][ny][nx]; overwritten with
 *      the per-shot gradients sum_n lambda^{n+1} Ey^n and
 *      sum_n lambda^{n+1} curlH^n on the interior window, 0 elsewhere.
 *      Either may be NULL.
 */
tm_status tm_adjoint(tm_plan* plan, void* ws, uint64_t ws_bytes, const float* ca,
                     const float* cb, const float* cq, const float* f, const float* grad_r,
                     float* grad_f, float* grad_ca_shot, float* grad_cb_shot, void* stream);

/*
 * Shot sum of the per-shot gradients: grad[j] = sum_s
 * grad_shot[s][j], shots summed in ascending order (deterministic).
 * Defined by: the page's kernel combine_grad, launched at the end of
 * backward over the per-shot gradient workspace.
 * grad_ca/grad_cb: device float32 [ny][nx], overwritten.  A NULL pair
 * member is skipped.  (With model_per_shot each shot's gradient belongs to
 * its own model and is used as it is; the sum is still computed if asked.)
 */
tm_status tm_grad(const tm_plan* plan, const float* grad_ca_shot, const float* grad_cb_shot,
                  float* grad_ca, float* grad_cb, void* stream);

/*
 * Gradients in the physical parameters by the chain rule
 * (defined by the page's kernel convert_grad_ca_cb_to_eps_sigma: its
 * closed forms in Ca, Cb and dt, and the EP0 value it defines): with eps = EP0 eps_r (EP0 =
 * 8.8541878128e-12 F/m) and s = sigma dt / (2 eps), the update
 * coefficients are Ca = (1 - s) / (1 + s) and Cb = (dt / eps) / (1 + s), so
 *   dJ/deps_r  = EP0 (dJ/dCa (1 - Ca) Cb / dt - dJ/dCb Cb^2 / dt),
 *   dJ/dsigma  = -dJ/dCa (1 + Ca) Cb / 2 - dJ/dCb Cb^2 / 2,
 * per cell, in float32.  Cq (the magnetic coefficient) is not involved.
 *   ca, cb: device float32 [ny][nx], the coefficients the gradients were
 *      taken at (required).  With model_per_shot, call it once per shot
 *      with that shot's coefficients and gradients.
 *   grad_ca, grad_cb: device float32 [ny][nx] (e.g. tm_grad's outputs); a
 *      NULL input counts as zero.
 *   dt: the time step (seconds) the coefficients were built with; must be
 *      finite and > 0 (TM_EINVAL otherwise).
 *   grad_eps_r, grad_sigma: device float32 [ny][nx], overwritten; a NULL
 *      output is skipped (both NULL: nothing is launched).
 * The result is exact for coefficients of the form above; for other Ca/Cb
 * it is the chain rule of that form evaluated at the given values.
 */
tm_status tm_grad_eps_sigma(const tm_plan* plan, const float* ca, const float* cb,
                            const float* grad_ca, const float* grad_cb, double dt,
                            float* grad_eps_r, float* grad_sigma, void* stream);

/*
 * The FP8 snapshot encoding (TM_SNAP_FP8), defined by the page's
 * forward_kernel_e_with_storage_fp8 and its conversions fp8_e4m3_from_float /
 * fp8_e4m3_to_float, their intrinsic path: OCP E4M3 with saturation to the
 * largest finite value.  encode: float32 -> one
 * byte per element, round to nearest even, |x| > 448 -> +-448, NaN -> NaN;
 * decode: byte -> float32 (exact).  in/out: device arrays of n elements
 * (n >= 0; NULL allowed only for n == 0).  The same conversions are used
 * by the step kernels.
 */
tm_status tm_fp8_encode(const float* in, uint8_t* out, int64_t n, void* stream);
tm_status tm_fp8_decode(const uint8_t* in, float* out, int64_t n, void* stream);

/*
 * Kernel timing, a diagnostic for roofline figures.  With sampling on
 * (every > 0), every ``every``-th time step of tm_forward and tm_adjoint
 * brackets each of its stencil-kernel launches with a pair of HIP events
 * recorded on the call's stream; every = 0 turns sampling off.  Nothing else
 * changes: the same kernels run in the same order.
 */
tm_status tm_timing_enable(tm_plan* plan, int32_t every);

/*
 * Per-kernel sums of the sampled durations (milliseconds) and sample counts
 * since the previous read, for kernels 0 .. tm_kernel_count()-1, into
 * caller arrays of tm_kernel_count() entries; then clears them.  Waits for
 * the recorded events (host-blocking).
 */
tm_status tm_timing_read(tm_plan* plan, double* total_ms, int64_t* count);

/* Number of timed kernels, and the name of kernel ``k`` (the prefix of its
 * symbol name as profilers print it, with "_uq" for the two-step instances
 * that use one Cq value instead of reading the array and "_store" for the
 * forward launches that store snapshots; NULL when k is out of range). */
int32_t tm_kernel_count(void);
const char* tm_kernel_name(int32_t k);

/* Static description of a status code. */
const char* tm_status_string(tm_status status);

#ifdef __cplusplus
}
#endif

#endif /* TM_FDTD_H */
